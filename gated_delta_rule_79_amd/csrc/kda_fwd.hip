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
#include <algorithm>
#include <cstdlib>

#include "kda_internal.hpp"

#ifndef KDA_STATE_PF
#define KDA_STATE_PF 1
#endif

namespace kda {

// ---------------------------------------------------------------------------
// chunk map
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void kda_chunk_map(const int32_t* __restrict__ cu, int N, int T,
                                                     ChunkInfo* __restrict__ chunks,
                                                     int32_t* __restrict__ seq_chunk0, int max_chunks,
                                                     int32_t* __restrict__ seq_order) {
  constexpr int MAX_SORT = 4096;
  __shared__ int32_t part[1024];
  __shared__ int32_t nchk[MAX_SORT];
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
  // Sequences by decreasing chunk count (ties by index).  The sequential passes
  // take their units in this order, so the longest chains start first and the
  // shorter ones fill the compute units around them.
  if (N <= MAX_SORT) {
    for (int s = tid; s < N; s += 1024) nchk[s] = sc0[s + 1] - sc0[s];
    __syncthreads();
    for (int s = tid; s < N; s += 1024) {
      const int ns = nchk[s];
      int rank = 0;
      for (int s2 = 0; s2 < N; ++s2) rank += (nchk[s2] > ns) || (nchk[s2] == ns && s2 < s);
      seq_order[rank] = s;
    }
  } else {
    for (int s = tid; s < N; s += 1024) seq_order[s] = s;
  }
}

hipError_t launch_chunk_map(const Args& a, hipStream_t st) {
  KDA_TIMED("kda_chunk_map", st,
            hipLaunchKernelGGL(kda_chunk_map, dim3(1), dim3(1024), 0, st, a.cu, a.N, a.T, a.chunks, a.seq_chunk0,
                               a.max_chunks, a.seq_order));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// prep: chunk-parallel part
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV>
struct PrepLds {
  using OP = typename OpOf<E>::T;
  static constexpr int PE = PADE<E>, PO = PADE<OP>;
  static constexpr int LDG = DK + 4;   // float g[CH][LDG]
  static constexpr int LDK = DK + PE;  // E     k[CH][LDK]
  static constexpr int LDT = CH + PO;  // OP    x[*][LDT]
  static constexpr int LDA = CH + 4;   // float A[CH][LDA]
  static constexpr size_t G = 0;
  static constexpr size_t K = G + (size_t)CH * LDG * 4;
  static constexpr size_t KPT = K + (size_t)CH * LDK * sizeof(E);
  static constexpr size_t VT = KPT + (size_t)DK * LDT * sizeof(OP);
  static constexpr size_t A = VT + (size_t)DV * LDT * sizeof(OP);
  static constexpr size_t TOT = A + (size_t)CH * LDA * 4;
  static constexpr size_t BETA = TOT + 256 * 8;   // TOT: double [256 / DK][DK] part sums of the scan
  static constexpr size_t X = BETA + CH * 4;
  static constexpr size_t BYTES = X + 3 * 256 * 4;
  // aliases used once the Gram blocks are done
  static constexpr size_t T = G;     // float [CH][LDA]  (fits in g)
  static constexpr size_t TE = K;    // OP    [CH][LDT]  (fits in k)
  static_assert((size_t)CH * LDA * 4 <= (size_t)CH * LDG * 4, "T alias");
  static_assert((size_t)CH * LDT * sizeof(OP) <= (size_t)CH * LDK * sizeof(E), "Te alias");
  static_assert(BYTES <= 163840, "prep LDS");
  static_assert(TOT % 8 == 0, "fp64 scan partials stay 8-byte aligned");
};

// QKN: q and k rows are L2-normalised on load (KDA_FLAG_QK_L2NORM).
template <typename E, int DK, int DV, bool BWD, bool QKN>
__global__ __launch_bounds__(256) void kda_prep(const Args a) {
  using L = PrepLds<E, DK, DV>;
  using OP = typename L::OP;
  constexpr int NT = 256;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  const int j = blockIdx.x, h = blockIdx.y, H = a.H;
  const ChunkInfo ci = a.chunks[j];
  if (ci.len <= 0) return;
  const int len = ci.len;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), r16 = l & 15, q4 = l >> 4;

  float* sG = reinterpret_cast<float*>(smem + L::G);
  E* sK = reinterpret_cast<E*>(smem + L::K);
  OP* sKpT = reinterpret_cast<OP*>(smem + L::KPT);
  OP* sVT = reinterpret_cast<OP*>(smem + L::VT);
  float* sA = reinterpret_cast<float*>(smem + L::A);
  double* sTot = reinterpret_cast<double*>(smem + L::TOT);
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
  if (tid == 0) a.steep[blk] = 1;   // this kernel always forms its Gram blocks through 8-token groups
  OP* wW = reinterpret_cast<OP*>(a.wsW) + blk * WB::W;
  OP* wKhT = reinterpret_cast<OP*>(a.wsKhT) + blk * WB::KHT;
  OP* wQt = reinterpret_cast<OP*>(a.wsQt) + blk * WB::QT;
  OP* wUt = reinterpret_cast<OP*>(a.wsUt) + blk * WB::UT;
  OP* wAqk = reinterpret_cast<OP*>(a.wsAqk) + blk * WB::AQK;
  float* wGam = a.wsGam + blk * WB::GAM;

  // ---- 1. all global loads of the chunk are issued here, before any use, so
  // their latencies overlap.  Wave w loads token rows 16w..16w+15; lane
  // (r16, q4) holds 8 consecutive channels 32*ks + 8*q4 of row 16w + r16.
  constexpr int NKS = DK / 32, NVS = DV / 32;
  const int r = 16 * w + r16;
  const bool rv_ok = r < len;
  float xq[NKS][8], xk[NKS][8], xl[NKS][8], xv[NVS][8];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    load8<E>(qh + r * rk + 32 * ks + 8 * q4, rv_ok, xq[ks]);
    load8<E>(kh + r * rk + 32 * ks + 8 * q4, rv_ok, xk[ks]);
    load8<E>(lh + r * rk + 32 * ks + 8 * q4, rv_ok, xl[ks]);
  }
#pragma unroll
  for (int vs = 0; vs < NVS; ++vs) load8<E>(vh + r * rv + 32 * vs + 8 * q4, rv_ok, xv[vs]);
  if constexpr (QKN) {   // row r's channels sit in this lane and the lanes 16 and 32 away
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        sq += xq[ks][u] * xq[ks][u];
        sk += xk[ks][u] * xk[ks][u];
      }
    sq += __shfl_xor(sq, 16);
    sq += __shfl_xor(sq, 32);
    sk += __shfl_xor(sk, 16);
    sk += __shfl_xor(sk, 32);
    const float nq = 1.0f / sqrtf(sq + L2N_EPS), nk = 1.0f / sqrtf(sk + L2N_EPS);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        xq[ks][u] *= nq;   // this kernel serves fp32 inputs: the normalised rows stay exact
        xk[ks][u] *= nk;
      }
  }
  if (rv_ok) {   // rows past the chunk stay 0 (no decay)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int u = 0; u < 8; ++u) xl[ks][u] = floor_log_alpha(a.gate_ls ? logsigmoid(xl[ks][u]) : xl[ks][u]);
  }
  const float bet = tid < len ? f32(bh[(size_t)tid * H]) : 0.f;
  if (tid < CH) sBeta[tid] = bet;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int c0 = 32 * ks + 8 * q4;
    *reinterpret_cast<f32x4*>(sG + r * L::LDG + c0) = f32x4{xl[ks][0], xl[ks][1], xl[ks][2], xl[ks][3]};
    *reinterpret_cast<f32x4*>(sG + r * L::LDG + c0 + 4) = f32x4{xl[ks][4], xl[ks][5], xl[ks][6], xl[ks][7]};
    store4<E>(sK + r * L::LDK + c0, xk[ks][0], xk[ks][1], xk[ks][2], xk[ks][3]);
    store4<E>(sK + r * L::LDK + c0 + 4, xk[ks][4], xk[ks][5], xk[ks][6], xk[ks][7]);
  }
#pragma unroll
  for (int vs = 0; vs < NVS; ++vs)
#pragma unroll
    for (int i = 0; i < 8; ++i) sVT[(32 * vs + 8 * q4 + i) * L::LDT + r] = cvt<OP>(xv[vs][i]);
  __syncthreads();
  // cumulative sum over tokens, in place: thread (channel c, part s) scans RPS rows.
  // The sums are taken in fp64 and each g is rounded to fp32 once: under the log
  // alpha floor |g| reaches 64 * 16 within a chunk, where one fp32 rounding is
  // already 2^-14 (and the decayed factors carry the error of g as a relative one).
  {
    constexpr int NSPLIT = NT / DK, RPS = CH / NSPLIT;
    const int c = tid % DK, s = tid / DK;
    double tot = 0.0;
#pragma unroll 8
    for (int rr = s * RPS; rr < (s + 1) * RPS; ++rr) tot += (double)sG[rr * L::LDG + c];
    sTot[s * DK + c] = tot;
  }
  __syncthreads();
  {
    constexpr int NSPLIT = NT / DK, RPS = CH / NSPLIT;
    const int c = tid % DK, s = tid / DK;
    double acc = 0.0;
    for (int s2 = 0; s2 < s; ++s2) acc += sTot[s2 * DK + c];
#pragma unroll 8
    for (int rr = s * RPS; rr < (s + 1) * RPS; ++rr) {
      acc += (double)sG[rr * L::LDG + c];
      sG[rr * L::LDG + c] = (float)acc;
    }
  }
  __syncthreads();

  // ---- 2. elementwise: K+^T (LDS), Kh^T, Qt (own rows, from registers), Gamma_C
  {
    const int rr = tid & (CH - 1);
    for (int c = tid / CH; c < DK; c += NT / CH) {
      const float g = sG[rr * L::LDG + c];
      const float gl = sG[(CH - 1) * L::LDG + c];
      const float kv = f32(sK[rr * L::LDK + c]);
      sKpT[c * L::LDT + rr] = cvt<OP>(kv * __expf(g));
      wKhT[c * CH + rr] = cvt<OP>(kv * __expf(gl - g));
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int c0 = 32 * ks + 8 * q4;
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = xq[ks][i] * __expf(sG[r * L::LDG + c0 + i]);
      store4<OP>(wQt + r * DK + c0, y[0], y[1], y[2], y[3]);
      store4<OP>(wQt + r * DK + c0 + 4, y[4], y[5], y[6], y[7]);
    }
    for (int c = tid; c < DK; c += NT) wGam[c] = __expf(sG[(CH - 1) * L::LDG + c]);
    if constexpr (BWD) {
      // Kh token-major in fp32 (the reverse pass multiplies it as a split operand)
      float* wKhF = a.wsKhF + blk * WB::KHF;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int c0 = 32 * ks + 8 * q4;
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          y[i] = xk[ks][i] * __expf(sG[(CH - 1) * L::LDG + c0 + i] - sG[r * L::LDG + c0 + i]);
        *reinterpret_cast<f32x4*>(wKhF + r * DK + c0) = f32x4{y[0], y[1], y[2], y[3]};
        *reinterpret_cast<f32x4*>(wKhF + r * DK + c0 + 4) = f32x4{y[4], y[5], y[6], y[7]};
      }
    }
  }

  // ---- 3. decayed Gram blocks: wave w owns row block a = w.  Reference rows in the
  // middle of 8-token groups (group_ref): the lane's row r in group R carries
  // e^{g_r - g_m(R)}; the column operand of row group R (h = 0, 1 of the block)
  // carries e^{g_m(R) - g_i} for columns in groups up to R and zero beyond, so each
  // block is two products, one per row group.  The gated factors can exceed fp16
  // range, so they are split bf16 (fp32 inputs: fp32).
  {
    const int ab = w;
    const int ref = group_ref(r >> 3);
    using SE = typename std::conditional<sizeof(E) == 4, float, bf16>::type;
    SFrag<SE> fk[NKS], fq[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int c0 = 32 * ks + 8 * q4;
      float yq[8], yk[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float e = __expf(sG[r * L::LDG + c0 + i] - sG[ref * L::LDG + c0 + i]);
        yk[i] = xk[ks][i] * e;
        yq[i] = xq[ks][i] * e;
      }
      fk[ks] = sfrag_from<SE>(yk);
      fq[ks] = sfrag_from<SE>(yq);
    }
    for (int b = 0; b <= ab; ++b) {
      f32x4 akk[2] = {zero4(), zero4()}, aqk[2] = {zero4(), zero4()};
      const int i = 16 * b + r16, C = i >> 3;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int R = 2 * ab + hh, mr = group_ref(R);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const int c0 = 32 * ks + 8 * q4;
          float xr[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const float x = f32(sK[i * L::LDK + c0 + u]) * __expf(sG[mr * L::LDG + c0 + u] - sG[i * L::LDG + c0 + u]);
            xr[u] = C <= R ? x : 0.f;
          }
          const SFrag<SE> fr = sfrag_from<SE>(xr);
          akk[hh] = mma_ss(fk[ks], fr, akk[hh]);
          aqk[hh] = mma_ss(fq[ks], fr, aqk[hh]);
        }
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int rr = 16 * ab + 4 * q4 + ii, cc = 16 * b + r16;
        const float vk = (q4 >> 1) ? akk[1][ii] : akk[0][ii], vq = (q4 >> 1) ? aqk[1][ii] : aqk[0][ii];
        sA[rr * L::LDA + cc] = cc < rr ? sBeta[rr] * vk : 0.f;
        wAqk[rr * CH + cc] = cvt<OP>(cc <= rr ? vq : 0.f);
        if constexpr (BWD) a.wsG[blk * WB::G + rr * CH + cc] = cc < rr ? vk : 0.f;
      }
    }
    for (int b = ab + 1; b < 4; ++b) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int rr = 16 * ab + 4 * q4 + ii, cc = 16 * b + r16;
        sA[rr * L::LDA + cc] = 0.f;
        wAqk[rr * CH + cc] = cvt<OP>(0.f);
        if constexpr (BWD) a.wsG[blk * WB::G + rr * CH + cc] = 0.f;
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
  OP* sTe = reinterpret_cast<OP*>(smem + L::TE);
  for (int o = tid; o < CH * CH; o += NT) {
    const int rr = o / CH, cc = o % CH;
    const float t = sT[rr * L::LDA + cc];
    sTe[rr * L::LDT + cc] = cvt<OP>(t * sBeta[cc]);
    if constexpr (BWD) reinterpret_cast<OP*>(a.wsT)[blk * WB::TT + o] = cvt<OP>(t);   // an MFMA operand only
  }
  __syncthreads();
  {
    // W^T tiles: C'[ch][tok] = sum_i K+^T[ch][i] Te[tok][i]; lane gets W[tok][4 consecutive ch]
    constexpr int NTI = (CH / 16) * (DK / 16);
    for (int t = w; t < NTI; t += 4) {
      const int mt = t % (CH / 16), nt = t / (CH / 16);
      const f32x4 acc = tile_mm<CH>([&](int rr, int k) { return frag_row<OP>(sKpT, L::LDT, 16 * nt + rr, k); },
                                    [&](int rr, int k) { return frag_row<OP>(sTe, L::LDT, 16 * mt + rr, k); },
                                    zero4());
      store4<OP>(wW + (16 * mt + r16) * DK + 16 * nt + 4 * q4, acc[0], acc[1], acc[2], acc[3]);
    }
    // U~ tiles: C[tok][dv]; lane holds 4 consecutive tokens of one value column -> U~^T rows
    // (fp32 for the backward, where its rounding would reach the gradients)
    constexpr int NTU = (CH / 16) * (DV / 16);
    for (int t = w; t < NTU; t += 4) {
      const int mt = t % (CH / 16), nt = t / (CH / 16);
      const f32x4 acc = tile_mm<CH>([&](int rr, int k) { return frag_row<OP>(sTe, L::LDT, 16 * mt + rr, k); },
                                    [&](int rr, int k) { return frag_row<OP>(sVT, L::LDT, 16 * nt + rr, k); },
                                    zero4());
      if constexpr (BWD)
        *reinterpret_cast<f32x4*>(a.wsUtF + blk * WB::UTF + (16 * nt + r16) * CH + 16 * mt + 4 * q4) = acc;
      else
        store4<OP>(wUt + (16 * nt + r16) * CH + 16 * mt + 4 * q4, acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// prep for bf16 inputs: persistent, 8 waves
// ---------------------------------------------------------------------------
// One work-group per compute unit walks the chunk-heads item, item + grid, ...
// (item = chunk * H + head).  The inputs of the next item are loaded into
// registers while the current one is computed, so the loads overlap compute.
// Wave w: row block a = w & 3 of the Gram blocks, with the (a + 1) column
// blocks split between the two waves w and w + 4.  T = (I + A)^-1: the four
// diagonal 16x16 blocks by substitution in one wave (each lane keeps one
// column in registers, so no cross-lane traffic), then the off-diagonal
// blocks level by level with fp32 MFMA: T_ab = -T_aa sum_k A_ak T_kb.
template <int DK, int DV>
struct Prep8Lds {
  static constexpr int LDG = DK + 4;   // float [CH][LDG]  log_alpha, then g
  static constexpr int LDK = DK + 8;   // bf16  [CH][LDK]  k, q
  static constexpr int LDT = CH + 8;   // fp16  [*][LDT]   K+^T, V^T, Te
  static constexpr int LDA = CH + 4;   // float [CH][LDA]  A, T
  static constexpr size_t G = 0;
  static constexpr size_t K = G + (size_t)CH * LDG * 4;
  static constexpr size_t Q = K + (size_t)CH * LDK * 2;
  static constexpr size_t GKQ_END = Q + (size_t)CH * LDK * 2;
  // once the Gram blocks are done, T and Te take the place of g, k and q
  static constexpr size_t T = 0;
  static constexpr size_t TE = T + (size_t)CH * LDA * 4;
  static constexpr size_t TEL = TE + (size_t)CH * LDT * 2;    // lo half of Te (training mode)
  static_assert(TEL + (size_t)CH * LDT * 2 <= GKQ_END, "T, Te alias g, k, q");
  static constexpr size_t KPT = GKQ_END;                      // fp16  [DK][LDT]
  static constexpr size_t VT = KPT + (size_t)DK * LDT * 2;    // fp16  [DV][LDT]
  static constexpr size_t A = VT + (size_t)DV * LDT * 2;      // float [CH][LDA]  beta * strict Gram
  static constexpr size_t X = A + (size_t)CH * LDA * 4;       // float [3][256]   off-diagonal partial sums
  static constexpr size_t BETA = X + 3 * 256 * 4;             // float [CH]
  static constexpr size_t RED = BETA + CH * 4;                // float [512]
  static constexpr size_t NRM = RED + 512 * 4;                // float [2][CH]  1/|q_r|, 1/|k_r| (QKN)
  // decayed Gram blocks, one pass of GC channels at a time:
  static constexpr int GC = 32;
  static constexpr int LDQ = GC + 8;                          // bf16 [CH][LDQ]  k~, q~ (hi, lo)
  static constexpr int LDR = GC + 4;                          // float [CH][LDR] k e^{g_m - g}
  static constexpr size_t GKH = NRM + 2 * CH * 4;
  static constexpr size_t GKL = GKH + (size_t)CH * LDQ * 2;
  static constexpr size_t GQH = GKL + (size_t)CH * LDQ * 2;
  static constexpr size_t GQL = GQH + (size_t)CH * LDQ * 2;
  static constexpr size_t GKR = GQL + (size_t)CH * LDQ * 2;
  static constexpr size_t GF = GKR + (size_t)CH * LDR * 4;   // float [28][GC] e^{g_m(R) - g_m(C)}, C < R
  static constexpr size_t BYTES = GF + NGROUP_PAIRS * GC * 4;
  static_assert(BYTES <= 163840, "prep LDS");
  static_assert(GKH % 16 == 0 && GKR % 16 == 0 && GF % 16 == 0, "16-byte rows");
};

// C(16x16) += A(16x16) B(16x16), fp32 operands in LDS (row-major), fp32 MFMA.
// Lane (r16, q4) supplies A[r16][4q4 + m] and B[4q4 + m][r16] to MFMA m.
__device__ __forceinline__ f32x4 mm16_f32(const float* A, int lda, const float* B, int ldb, f32x4 c) {
  const int l = lane_id(), r16 = l & 15, q4 = l >> 4;
  const f32x4 av = *reinterpret_cast<const f32x4*>(A + r16 * lda + 4 * q4);
#pragma unroll
  for (int m = 0; m < 4; ++m) c = __builtin_amdgcn_mfma_f32_16x16x4f32(av[m], B[(4 * q4 + m) * ldb + r16], c, 0, 0, 0);
  return c;
}

// The chunk's V rows ([64][DV] bf16, row pitch ld) for V^T in LDS: a thread loads rows
// 2p and 2p + 1 of one 8-column piece and writes the eight (row 2p, row 2p + 1) pairs,
// converted to the operand type, as 4-byte words at V^T[col][2p]; the 32 lanes of a
// half-wave take the 32 row pairs of one piece, so their words fall in distinct banks.
// Rows >= nrows are not read (row 0 is re-read) and are stored as zeros.
template <int DV, int NT>
struct VPairs {
  static constexpr int NP = CH / 2, NI = NP * (DV / 8), PER = (NI + NT - 1) / NT;
  u32x4 r0[PER], r1[PER];
  __device__ __forceinline__ void load(const bf16* __restrict__ src, size_t ld, int nrows) {
    static_for<0, PER>([&](auto I) __attribute__((always_inline)) {
      const int v0 = threadIdx.x + I * NT, v = (NI % NT == 0 || v0 < NI) ? v0 : 0;
      const int p = v % NP, cp = v / NP;
      const int ra = 2 * p < nrows ? 2 * p : 0, rb = 2 * p + 1 < nrows ? 2 * p + 1 : 0;
      r0[I] = *reinterpret_cast<const u32x4*>(src + (size_t)ra * ld + 8 * cp);
      r1[I] = *reinterpret_cast<const u32x4*>(src + (size_t)rb * ld + 8 * cp);
    });
  }
  template <typename OP>
  __device__ __forceinline__ void store_t(OP* dst, int dst_ld, int nrows) const {
    static_assert(sizeof(OP) == 2, "pairs of 2-byte elements");
    static_for<0, PER>([&](auto I) __attribute__((always_inline)) {
      const int v = threadIdx.x + I * NT;
      if (NI % NT == 0 || v < NI) {
        const int p = v % NP, cp = v / NP;
        const bool oka = 2 * p < nrows, okb = 2 * p + 1 < nrows;
        const bf16* a = reinterpret_cast<const bf16*>(&r0[I]);
        const bf16* b = reinterpret_cast<const bf16*>(&r1[I]);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const OP x = cvt<OP>(oka ? f32(a[u]) : 0.f), y = cvt<OP>(okb ? f32(b[u]) : 0.f);
          *reinterpret_cast<uint32_t*>(dst + (8 * cp + u) * dst_ld + 2 * p) =
              (uint32_t)__builtin_bit_cast(unsigned short, x) | ((uint32_t)__builtin_bit_cast(unsigned short, y) << 16);
        }
      }
    });
  }
};

// GATE: log_alpha holds a raw gate x (KDA_FLAG_GATE_LOGSIGMOID).  Both options
// are compile-time so the plain kernel keeps its register budget.
// PATH 0: the usual chunk-heads; a chunk-head where some channel decays by more than
// e^-STEEP_SPAN within 8 tokens is flagged in a.steep and left for PATH 1, which
// visits only the flagged ones and forms the decayed Gram blocks through 8-token
// groups (see group_ref).  Two instantiations keep the usual path's registers free of
// the other one's.
template <int DK, int DV, bool BWD, bool QKN, bool GATE, int PATH>
__global__ __launch_bounds__(512) void kda_prep8(const Args a) {
  using L = Prep8Lds<DK, DV>;
  using E = bf16;
  using OP = f16;
  using WB = WsBlock<E, DK, DV>;
  constexpr int NT = 512, NKS = DK / 32;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), r16 = l & 15, q4 = l >> 4;
  const int H = a.H;
  const int n_items = a.max_chunks * H;
  const size_t rk = (size_t)H * DK, rv = (size_t)H * DV;

  float* sG = reinterpret_cast<float*>(smem + L::G);
  E* sK = reinterpret_cast<E*>(smem + L::K);
  E* sQ = reinterpret_cast<E*>(smem + L::Q);
  float* sT = reinterpret_cast<float*>(smem + L::T);
  OP* sTe = reinterpret_cast<OP*>(smem + L::TE);
  OP* sTeL = reinterpret_cast<OP*>(smem + L::TEL);
  OP* sKpT = reinterpret_cast<OP*>(smem + L::KPT);
  OP* sVT = reinterpret_cast<OP*>(smem + L::VT);
  float* sA = reinterpret_cast<float*>(smem + L::A);
  float* sX = reinterpret_cast<float*>(smem + L::X);
  float* sBeta = reinterpret_cast<float*>(smem + L::BETA);
  float* sRed = reinterpret_cast<float*>(smem + L::RED);
  // row scales of q and k: 1/|row| with KDA_FLAG_QK_L2NORM (the raw rows stay in
  // LDS and every use multiplies by the scale, so normalisation adds no rounding)
  float* sNq = reinterpret_cast<float*>(smem + L::NRM);
  float* sNk = sNq + CH;
  auto nq = [&](int r) __attribute__((always_inline)) { if constexpr (QKN) return sNq[r]; else return 1.f; };
  auto nk = [&](int r) __attribute__((always_inline)) { if constexpr (QKN) return sNk[r]; else return 1.f; };

  const E* gq = reinterpret_cast<const E*>(a.q);
  const E* gk = reinterpret_cast<const E*>(a.k);
  const E* gl = reinterpret_cast<const E*>(a.la);
  const E* gv = reinterpret_cast<const E*>(a.v);
  const E* gb = reinterpret_cast<const E*>(a.beta);

  TileCopy<E, CH, DK, NT> pq, pk, pl;
  VPairs<DV, NT> pv;
  E pb = E(0.f);
  // The loads are issued without a branch and their values are not touched until the
  // next item is staged: a value used at once (or a load inside a branch) makes the
  // wave wait for every load and store it still has in flight.
  auto fetch = [&](int item, const ChunkInfo& c) __attribute__((always_inline)) {
    const int h = item % H;
    const size_t t0 = (size_t)c.t0;
    pq.load(gq + t0 * rk + (size_t)h * DK, rk, c.len);
    pk.load(gk + t0 * rk + (size_t)h * DK, rk, c.len);
    pl.load(gl + t0 * rk + (size_t)h * DK, rk, c.len);
    pv.load(gv + t0 * rv + (size_t)h * DV, rv, c.len);
    pb = gb[(t0 + (size_t)min(tid % CH, c.len - 1)) * H + h];   // rows past len: zeroed when staged
  };
  // The chunk record (t0, len) of each item is read one item before its inputs, through
  // a lane-varying offset that is always zero, so it stays in vector registers until the
  // fetch makes scalars of it (a uniform load is moved to scalar registers at once, and
  // that move waits for every load and store in flight).  Slot 0 always exists.
  struct Rec {
    int t0, len;
    bool valid;
  };
  auto record = [&](int it) __attribute__((always_inline)) {
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    const bool valid = it < n_items;
    const ChunkInfo* c = a.chunks + (valid ? it / H : 0) + z;
    return Rec{c->t0, c->len, valid};
  };
  auto chunk_of = [&](const Rec& r) __attribute__((always_inline)) {
    return r.valid ? ChunkInfo{0, __builtin_amdgcn_readfirstlane(r.t0), __builtin_amdgcn_readfirstlane(r.len), 0}
                   : ChunkInfo{0, 0, 0, 0};
  };

  // PATH 1 walks only the flagged items (the slots past the last chunk, never flagged
  // by PATH 0, are empty and end the walk wherever they are met).  The work-group looks
  // at 512 of its items at once: each thread reads one flag, and the first flagged one
  // (wave ballots, then the lowest wave) is the next item.
  const int32_t* steep = a.steep;
  __shared__ int sFirst[NT / 64];
  auto advance = [&](int it) __attribute__((always_inline)) {
    if constexpr (PATH == 1) {
      const long long G = gridDim.x;
      while (it < n_items) {
        const long long c = (long long)it + (long long)tid * G;
        const unsigned long long b = __ballot(c < n_items && steep[c] != 0);
        if (lane_id() == 0) sFirst[wave_id()] = b ? __ffsll((long long)b) - 1 : 64;
        __syncthreads();
        int first = -1;
#pragma unroll
        for (int ww = NT / 64 - 1; ww >= 0; --ww)
          if (sFirst[ww] < 64) first = ww * 64 + sFirst[ww];
        __syncthreads();
        if (first >= 0) return (int)(it + first * G);
        it = (int)std::min<long long>((long long)it + NT * G, n_items);
      }
    }
    return it;
  };
  int item = advance((int)blockIdx.x);
  ChunkInfo ci = chunk_of(record(item));
  if (ci.len > 0) fetch(item, ci);
  int nitem = ci.len > 0 ? advance(item + (int)gridDim.x) : n_items;
  Rec nrec = record(nitem);
  while (ci.len > 0) {   // the same value in every thread
    const size_t blk = (size_t)item;   // == chunk * H + head
    const int len = ci.len;
    OP* wW = reinterpret_cast<OP*>(a.wsW) + blk * WB::W;
    OP* wKhT = reinterpret_cast<OP*>(a.wsKhT) + blk * WB::KHT;
    OP* wQt = reinterpret_cast<OP*>(a.wsQt) + blk * WB::QT;
    OP* wAqk = reinterpret_cast<OP*>(a.wsAqk) + blk * WB::AQK;
    float* wGam = a.wsGam + blk * WB::GAM;

    __syncthreads();  // the previous item's LDS reads are done
    if constexpr (QKN) {
      float scq[decltype(pq)::PER], sck[decltype(pk)::PER];
      pq.row_inv_norms(L2N_EPS, scq);
      pk.row_inv_norms(L2N_EPS, sck);
#pragma unroll
      for (int I = 0; I < decltype(pq)::PER; ++I) {
        int row;
        if (pq.row_leader(I, row)) {
          sNq[row] = scq[I];
          sNk[row] = sck[I];
        }
      }
    }
    pk.template store_cvt<E>(sK, L::LDK, len);
    pq.template store_cvt<E>(sQ, L::LDK, len);
    if constexpr (GATE)   // raw gate x -> log alpha = logsigmoid(x)
      pl.template store_map<float>(sG, L::LDG, len, [](float x) { return floor_log_alpha(logsigmoid(x)); });
    else
      pl.template store_map<float>(sG, L::LDG, len, [](float x) { return floor_log_alpha(x); });
    pv.template store_t<OP>(sVT, L::LDT, len);   // V^T
    if (tid < CH) sBeta[tid] = tid < len ? f32(pb) : 0.f;
    const ChunkInfo nci = chunk_of(nrec);
    if (nci.len > 0) fetch(nitem, nci);
    const int n2item = nci.len > 0 ? advance(nitem + (int)gridDim.x) : n_items;
    const Rec n2rec = record(n2item);
    __syncthreads();

    // ---- cumulative sum of log_alpha over the chunk (per channel, NT / DK row parts)
    constexpr int NSPLIT = NT / DK, RPS = CH / NSPLIT;
    {
      const int c = tid % DK, s = tid / DK;
      float acc = 0.f;
#pragma unroll
      for (int rr = s * RPS; rr < (s + 1) * RPS; ++rr) {
        acc += sG[rr * L::LDG + c];
        sG[rr * L::LDG + c] = acc;
      }
      sRed[s * DK + c] = acc;
    }
    __syncthreads();
    {
      const int c = tid % DK, s = tid / DK;
      float off = 0.f;
      for (int s2 = 0; s2 < s; ++s2) off += sRed[s2 * DK + c];
#pragma unroll
      for (int rr = s * RPS; rr < (s + 1) * RPS; ++rr) sG[rr * L::LDG + c] += off;
    }
    __syncthreads();
    bool skip = false;
    if constexpr (PATH == 0) {
      skip = __syncthreads_or(steep_block(sG, L::LDG, tid, DK));
      if (tid == 0) a.steep[blk] = skip ? 1 : 0;
    }
    if (!skip) {

    // ---- elementwise: Qt (token rows), K+^T to LDS and Kh^T (channel rows), Gamma_C
    {
      constexpr int VA = DK / 8;   // 8-channel pieces per token row
#pragma unroll
      for (int i = 0; i < CH * VA / NT; ++i) {
        const int v = tid + i * NT, r = v / VA, c0 = (v % VA) * 8;
        float y[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) y[u] = f32(sQ[r * L::LDK + c0 + u]) * nq(r) * __expf(sG[r * L::LDG + c0 + u]);
        store4<OP>(wQt + r * DK + c0, y[0], y[1], y[2], y[3]);
        store4<OP>(wQt + r * DK + c0 + 4, y[4], y[5], y[6], y[7]);
        if constexpr (BWD) {
          // Kh token-major as a split pair of fp16 arrays (hi, then lo), the form in
          // which the reverse pass multiplies it
          OP* wKhH = reinterpret_cast<OP*>(a.wsKhF + blk * WB::KHF);
          OP* wKhL = wKhH + CH * DK;
#pragma unroll
          for (int u = 0; u < 8; ++u)
            y[u] = f32(sK[r * L::LDK + c0 + u]) * nk(r) * __expf(sG[(CH - 1) * L::LDG + c0 + u] - sG[r * L::LDG + c0 + u]);
          store4_split<OP>(wKhH + r * DK + c0, wKhL + r * DK + c0, y[0], y[1], y[2], y[3]);
          store4_split<OP>(wKhH + r * DK + c0 + 4, wKhL + r * DK + c0 + 4, y[4], y[5], y[6], y[7]);
        }
      }
#pragma unroll
      for (int i = 0; i < DK * (CH / 8) / NT; ++i) {
        const int v = tid + i * NT, c = v / (CH / 8), t0 = (v % (CH / 8)) * 8;
        const float glast = sG[(CH - 1) * L::LDG + c];
        float kp[8], kh[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float g = sG[(t0 + u) * L::LDG + c], kv = f32(sK[(t0 + u) * L::LDK + c]) * nk(t0 + u);
          kp[u] = kv * __expf(g);
          kh[u] = kv * __expf(glast - g);
        }
        store4<OP>(sKpT + c * L::LDT + t0, kp[0], kp[1], kp[2], kp[3]);
        store4<OP>(sKpT + c * L::LDT + t0 + 4, kp[4], kp[5], kp[6], kp[7]);
        if constexpr (BWD) {   // training mode: split, for the state update (see StateLds)
          OP* wKhTL = reinterpret_cast<OP*>(a.wsKhTL) + blk * WB::KHT;
          store4_split<OP>(wKhT + c * CH + t0, wKhTL + c * CH + t0, kh[0], kh[1], kh[2], kh[3]);
          store4_split<OP>(wKhT + c * CH + t0 + 4, wKhTL + c * CH + t0 + 4, kh[4], kh[5], kh[6], kh[7]);
        } else {
          store4<OP>(wKhT + c * CH + t0, kh[0], kh[1], kh[2], kh[3]);
          store4<OP>(wKhT + c * CH + t0 + 4, kh[4], kh[5], kh[6], kh[7]);
        }
      }
      if (tid < DK) wGam[tid] = __expf(sG[(CH - 1) * L::LDG + tid]);
    }

    // ---- decayed Gram blocks.  Usual chunks: reference rows in the middle of 16-row
    // blocks, one product per tile.  Chunks where some channel decays by more than
    // e^-32 within 8 tokens take the 8-token-group path, whose factors stay bounded
    // for any gate (see group_ref and CHAIN_MIN).
    if constexpr (PATH == 0) {
      // ---- decayed Gram blocks (split bf16 operands; reference row m(b) = 16b + 8).
      // Block (a, b), b <= a, of K+ K-^T is sum_c k~_r[c] (k_i[c] e^{g_m(b) - g_i}) e^{g_m(a) - g_m(b)}
      // with k~_r = k_r e^{g_r - g_m(a)}; every factor stays within an 8-token decay.  The
      // channels go in passes of GC: each pass tabulates k~ and q~ (split), k e^{g_m - g} and
      // the block-to-block factors once, and every wave reads its operands as 16-byte rows.
      // The ten blocks are dealt to the waves so each SIMD (waves w and w + 4) gets two or three.
      {
        constexpr int GC = L::GC, NPASS = DK / GC;
        bf16* tKh = reinterpret_cast<bf16*>(smem + L::GKH);
        bf16* tKl = reinterpret_cast<bf16*>(smem + L::GKL);
        bf16* tQh = reinterpret_cast<bf16*>(smem + L::GQH);
        bf16* tQl = reinterpret_cast<bf16*>(smem + L::GQL);
        float* tKR = reinterpret_cast<float*>(smem + L::GKR);
        float* tF = reinterpret_cast<float*>(smem + L::GF);
        // this wave's blocks: list index w and w + 8 of (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3)
        constexpr uint64_t BA = pack2({0, 1, 1, 2, 2, 2, 3, 3, 3, 3});
        constexpr uint64_t BB = pack2({0, 0, 1, 0, 1, 2, 0, 1, 2, 3});
        const int wu = __builtin_amdgcn_readfirstlane(w);   // wave-uniform, so the block choice is scalar
        const int nblk = wu < 2 ? 2 : 1;
        f32x4 akk[2] = {zero4(), zero4()}, aqk[2] = {zero4(), zero4()};
        static_assert(NT == CH * (GC / 4), "table build: one thread per (token, 4 channels)");
        for (int ps = 0; ps < NPASS; ++ps) {
          if (ps > 0) __syncthreads();   // the previous pass's table reads are done
          {
            const int r = tid / (GC / 4), cl0 = 4 * (tid % (GC / 4)), c0 = GC * ps + cl0;
            const int mref = 16 * (r >> 4) + 8;
            float ek[4], eq[4], kr[4];
  #pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float g = sG[r * L::LDG + c0 + u], gm = sG[mref * L::LDG + c0 + u];
              const float e = __expf(g - gm);
              const float kv = f32(sK[r * L::LDK + c0 + u]) * nk(r);
              ek[u] = kv * e;
              eq[u] = f32(sQ[r * L::LDK + c0 + u]) * nq(r) * e;
              kr[u] = kv * __expf(gm - g);
            }
            store4_split<bf16>(tKh + r * L::LDQ + cl0, tKl + r * L::LDQ + cl0, ek[0], ek[1], ek[2], ek[3]);
            store4_split<bf16>(tQh + r * L::LDQ + cl0, tQl + r * L::LDQ + cl0, eq[0], eq[1], eq[2], eq[3]);
            *reinterpret_cast<f32x4*>(tKR + r * L::LDR + cl0) = f32x4{kr[0], kr[1], kr[2], kr[3]};
            if (tid < 6 * GC) {   // pair (a, b), b < a, in the order (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
              const int pi = tid / GC, c = GC * ps + tid % GC;
              const int pa = pi < 1 ? 1 : (pi < 3 ? 2 : 3), pb = pi < 1 ? 0 : (pi < 3 ? pi - 1 : pi - 3);
              tF[tid] = __expf(sG[(16 * pa + 8) * L::LDG + c] - sG[(16 * pb + 8) * L::LDG + c]);
            }
          }
          __syncthreads();
  #pragma unroll
          for (int j = 0; j < 2; ++j) {
            if (j < nblk) {
              const int li = wu + 8 * j, ba = unpack2(BA, li), bb = unpack2(BB, li);
              const SFrag<bf16> fk = sfrag_pair<bf16>(tKh, tKl, L::LDQ, 16 * ba + r16, 8 * q4);
              const SFrag<bf16> fq = sfrag_pair<bf16>(tQh, tQl, L::LDQ, 16 * ba + r16, 8 * q4);
              const f32x4 v0 = *reinterpret_cast<const f32x4*>(tKR + (16 * bb + r16) * L::LDR + 8 * q4);
              const f32x4 v1 = *reinterpret_cast<const f32x4*>(tKR + (16 * bb + r16) * L::LDR + 8 * q4 + 4);
              float xr[8];
              if (bb == ba) {
  #pragma unroll
                for (int u = 0; u < 4; ++u) {
                  xr[u] = v0[u];
                  xr[u + 4] = v1[u];
                }
              } else {
                const float* f = tF + GC * (ba * (ba - 1) / 2 + bb) + 8 * q4;
                const f32x4 f0 = *reinterpret_cast<const f32x4*>(f), f1 = *reinterpret_cast<const f32x4*>(f + 4);
  #pragma unroll
                for (int u = 0; u < 4; ++u) {
                  xr[u] = v0[u] * f0[u];
                  xr[u + 4] = v1[u] * f1[u];
                }
              }
              const SFrag<bf16> fr = sfrag_from<bf16>(xr);
              akk[j] = mma_ss(fk, fr, akk[j]);
              aqk[j] = mma_ss(fq, fr, aqk[j]);
            }
          }
        }
  #pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (j < nblk) {
            const int li = wu + 8 * j, ba = unpack2(BA, li), bb = unpack2(BB, li);
  #pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
              const int rr = 16 * ba + 4 * q4 + ii, cc = 16 * bb + r16;
              sA[rr * L::LDA + cc] = cc < rr ? sBeta[rr] * akk[j][ii] : 0.f;
              wAqk[rr * CH + cc] = cvt<OP>(cc <= rr ? aqk[j][ii] : 0.f);
              if constexpr (BWD) a.wsG[blk * WB::G + rr * CH + cc] = cc < rr ? akk[j][ii] : 0.f;
            }
          }
        }
        if (w < 6) {   // blocks above the diagonal: (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
          const int ba = w < 3 ? 0 : (w < 5 ? 1 : 2), bb = w < 3 ? w + 1 : (w < 5 ? w - 1 : 3);
  #pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int rr = 16 * ba + 4 * q4 + ii, cc = 16 * bb + r16;
            sA[rr * L::LDA + cc] = 0.f;
            wAqk[rr * CH + cc] = cvt<OP>(0.f);
            if constexpr (BWD) a.wsG[blk * WB::G + rr * CH + cc] = 0.f;
          }
        }
      }
    } else {
      // ---- decayed Gram blocks (split bf16 operands; reference rows in the middle of
      // 8-token groups, m(R) = 8R + 4).  For row r in group R and column i in group C <= R,
      //   e^{g_r - g_i} = e^{g_r - g_m(R)} e^{g_m(R) - g_m(C)} e^{g_m(C) - g_i},
      // the outer two factors tabulated per (token, channel), the middle one per (R, C) pair.
      // With log alpha >= -LOG_ALPHA_FLOOR no factor exceeds e^{4 LOG_ALPHA_FLOOR}: the row
      // and column factors span at most 4 and 3 tokens and the chain factor is at most 1.
      // A 16x16 tile (a, b) is computed once per row group R in {2a, 2a+1} with the chain
      // folded into the column operand (zero for C > R, where the pairs lie above the
      // diagonal); each lane keeps the rows of its own group.  The channels go in passes of
      // GC; the 20 tile halves are dealt to the waves so each SIMD gets five.
      {
        constexpr int GC = L::GC, NPASS = DK / GC;
        bf16* tKh = reinterpret_cast<bf16*>(smem + L::GKH);
        bf16* tKl = reinterpret_cast<bf16*>(smem + L::GKL);
        bf16* tQh = reinterpret_cast<bf16*>(smem + L::GQH);
        bf16* tQl = reinterpret_cast<bf16*>(smem + L::GQL);
        float* tKR = reinterpret_cast<float*>(smem + L::GKR);
        float* tF = reinterpret_cast<float*>(smem + L::GF);
        // tile halves (a, b, h): list index w, w + 8, w + 16 for wave w
        constexpr uint64_t HA = pack2({0, 1, 1, 1, 2, 2, 2, 2, 2, 3, 3, 3, 3, 3, 3, 3, 0, 1, 2, 3});
        constexpr uint64_t HB = pack2({0, 0, 1, 0, 0, 1, 2, 0, 1, 0, 1, 2, 3, 0, 1, 2, 0, 1, 2, 3});
        constexpr uint64_t HH = pack2({1, 0, 1, 1, 0, 0, 1, 1, 1, 0, 0, 0, 1, 1, 1, 1, 0, 0, 0, 0});
        const int wu = __builtin_amdgcn_readfirstlane(w);   // wave-uniform, so the tile choice is scalar
        const int nitem = wu < 4 ? 3 : 2;
        f32x4 akk[3] = {zero4(), zero4(), zero4()}, aqk[3] = {zero4(), zero4(), zero4()};
        static_assert(NT == CH * (GC / 4), "table build: one thread per (token, 4 channels)");
        for (int ps = 0; ps < NPASS; ++ps) {
          if (ps > 0) __syncthreads();   // the previous pass's table reads are done
          {
            const int r = tid / (GC / 4), cl0 = 4 * (tid % (GC / 4)), c0 = GC * ps + cl0;
            const int mref = group_ref(r >> 3);
            float ek[4], eq[4], kr[4];
  #pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float g = sG[r * L::LDG + c0 + u], gm = sG[mref * L::LDG + c0 + u];
              const float kv = f32(sK[r * L::LDK + c0 + u]) * nk(r);
              const float e = __expf(g - gm);
              ek[u] = kv * e;
              eq[u] = f32(sQ[r * L::LDK + c0 + u]) * nq(r) * e;
              kr[u] = kv * __expf(gm - g);
            }
            store4_split<bf16>(tKh + r * L::LDQ + cl0, tKl + r * L::LDQ + cl0, ek[0], ek[1], ek[2], ek[3]);
            store4_split<bf16>(tQh + r * L::LDQ + cl0, tQl + r * L::LDQ + cl0, eq[0], eq[1], eq[2], eq[3]);
            *reinterpret_cast<f32x4*>(tKR + r * L::LDR + cl0) = f32x4{kr[0], kr[1], kr[2], kr[3]};
            for (int e = tid; e < NGROUP_PAIRS * GC; e += NT) {   // chain factors of the group pairs C < R
              const int pi = e / GC, c = GC * ps + e % GC;
              tF[e] = __expf(sG[group_ref(pair_r(pi)) * L::LDG + c] - sG[group_ref(pair_c(pi)) * L::LDG + c]);
            }
          }
          __syncthreads();
  #pragma unroll
          for (int j = 0; j < 3; ++j) {
            if (j < nitem) {
              const int li = wu + 8 * j, ba = unpack2(HA, li), bb = unpack2(HB, li), R = 2 * ba + unpack2(HH, li);
              const int C = 2 * bb + (r16 >> 3);   // group of this lane's column
              const SFrag<bf16> fk = sfrag_pair<bf16>(tKh, tKl, L::LDQ, 16 * ba + r16, 8 * q4);
              const SFrag<bf16> fq = sfrag_pair<bf16>(tQh, tQl, L::LDQ, 16 * ba + r16, 8 * q4);
              const f32x4 v0 = *reinterpret_cast<const f32x4*>(tKR + (16 * bb + r16) * L::LDR + 8 * q4);
              const f32x4 v1 = *reinterpret_cast<const f32x4*>(tKR + (16 * bb + r16) * L::LDR + 8 * q4 + 4);
              float xr[8];
              bool tiny = false;
              if (C < R) {
                const float* f = tF + GC * pair_index(R, C) + 8 * q4;
                const f32x4 f0 = *reinterpret_cast<const f32x4*>(f), f1 = *reinterpret_cast<const f32x4*>(f + 4);
  #pragma unroll
                for (int u = 0; u < 4; ++u) {
                  xr[u] = v0[u] * f0[u];
                  xr[u + 4] = v1[u] * f1[u];
                  tiny |= f0[u] < CHAIN_MIN || f1[u] < CHAIN_MIN;
                }
              } else {
                const bool on = C == R;   // C > R: pairs above the diagonal (zero, and kept finite)
  #pragma unroll
                for (int u = 0; u < 4; ++u) {
                  xr[u] = on ? v0[u] : 0.f;
                  xr[u + 4] = on ? v1[u] : 0.f;
                }
              }
              if (__any(tiny) && C < R) {   // one exponential per element (see CHAIN_MIN)
                const int i = 16 * bb + r16, c0 = GC * ps + 8 * q4, mr = group_ref(R);
  #pragma unroll
                for (int u = 0; u < 8; ++u)
                  xr[u] = f32(sK[i * L::LDK + c0 + u]) * nk(i) * __expf(sG[mr * L::LDG + c0 + u] - sG[i * L::LDG + c0 + u]);
              }
              const SFrag<bf16> fr = sfrag_from<bf16>(xr);
              akk[j] = mma_ss(fk, fr, akk[j]);
              aqk[j] = mma_ss(fq, fr, aqk[j]);
            }
          }
        }
  #pragma unroll
        for (int j = 0; j < 3; ++j) {
          if (j < nitem) {
            const int li = wu + 8 * j, ba = unpack2(HA, li), bb = unpack2(HB, li), hh = unpack2(HH, li);
            if ((q4 >> 1) == hh) {   // this lane's rows 4q4 .. 4q4 + 3 of the tile are in row group 2a + hh
  #pragma unroll
              for (int ii = 0; ii < 4; ++ii) {
                const int rr = 16 * ba + 4 * q4 + ii, cc = 16 * bb + r16;
                sA[rr * L::LDA + cc] = cc < rr ? sBeta[rr] * akk[j][ii] : 0.f;
                wAqk[rr * CH + cc] = cvt<OP>(cc <= rr ? aqk[j][ii] : 0.f);
                if constexpr (BWD) a.wsG[blk * WB::G + rr * CH + cc] = cc < rr ? akk[j][ii] : 0.f;
              }
            }
          }
        }
        if (w < 6) {   // blocks above the diagonal: (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
          const int ba = w < 3 ? 0 : (w < 5 ? 1 : 2), bb = w < 3 ? w + 1 : (w < 5 ? w - 1 : 3);
  #pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int rr = 16 * ba + 4 * q4 + ii, cc = 16 * bb + r16;
            sA[rr * L::LDA + cc] = 0.f;
            wAqk[rr * CH + cc] = cvt<OP>(0.f);
            if constexpr (BWD) a.wsG[blk * WB::G + rr * CH + cc] = 0.f;
          }
        }
      }
    }
    __syncthreads();  // A complete; g, k, q are dead (T and Te reuse their space)

    // ---- T = (I + A)^-1
    if (w == 0) {
      // diagonal blocks: lane (block bb, column c) keeps column c of T_bb in registers
      const int bb = l >> 4, c = l & 15;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float* nrow = sA + (16 * bb + r) * L::LDA + 16 * bb;
        float s = 0.f;
#pragma unroll
        for (int i4 = 0; i4 < r; i4 += 4) {
          const f32x4 nv = *reinterpret_cast<const f32x4*>(nrow + i4);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (i4 + u < r) s += nv[u] * x[i4 + u];
        }
        x[r] = r == c ? 1.f : (r > c ? -s : 0.f);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sT[(16 * bb + r) * L::LDA + 16 * bb + c] = x[r];
    } else {
      // blocks above the diagonal are zero
      for (int o = tid - 64; o < 6 * 256; o += NT - 64) {
        const int blkid = o >> 8, e = o & 255;
        const int ra = blkid < 3 ? 0 : (blkid < 5 ? 1 : 2);
        const int cb = blkid < 3 ? blkid + 1 : (blkid < 5 ? blkid - 1 : 3);
        sT[(16 * ra + (e >> 4)) * L::LDA + 16 * cb + (e & 15)] = 0.f;
      }
    }
    __syncthreads();
    for (int d = 1; d < 4; ++d) {
      const int nblk = 4 - d;
      if (w < nblk) {
        const int bc = w, ar = w + d;
        f32x4 x = zero4();
        for (int kb = bc; kb < ar; ++kb)
          x = mm16_f32(sA + 16 * ar * L::LDA + 16 * kb, L::LDA, sT + 16 * kb * L::LDA + 16 * bc, L::LDA, x);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sX[w * 256 + (4 * q4 + ii) * 16 + r16] = x[ii];
      }
      __syncthreads();
      if (w < nblk) {
        const int bc = w, ar = w + d;
        const f32x4 y = mm16_f32(sT + 16 * ar * L::LDA + 16 * ar, L::LDA, sX + w * 256, 16, zero4());
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sT[(16 * ar + 4 * q4 + ii) * L::LDA + 16 * bc + r16] = -y[ii];
      }
      __syncthreads();
    }

    // ---- Te = T diag(beta) in fp16; W = Te K+, U~ = Te V.  In training mode Te is a
    // split pair: W and U~ reach every saved state, whose rounding dlog alpha collects
    for (int o = tid; o < CH * CH / 4; o += NT) {
      const int rr = (4 * o) / CH, cc = (4 * o) % CH;
      const f32x4 t = *reinterpret_cast<const f32x4*>(sT + rr * L::LDA + cc);
      const float t0 = t[0] * sBeta[cc], t1 = t[1] * sBeta[cc + 1], t2 = t[2] * sBeta[cc + 2], t3 = t[3] * sBeta[cc + 3];
      if constexpr (BWD)
        store4_split<OP>(sTe + rr * L::LDT + cc, sTeL + rr * L::LDT + cc, t0, t1, t2, t3);
      else
        store4<OP>(sTe + rr * L::LDT + cc, t0, t1, t2, t3);
      if constexpr (BWD)   // the backward uses T only as an MFMA operand
        store4<OP>(reinterpret_cast<OP*>(a.wsT) + blk * WB::TT + rr * CH + cc, t[0], t[1], t[2], t[3]);
    }
    __syncthreads();
    {
      // W^T tiles: C'[ch][tok] = sum_i K+^T[ch][i] Te[tok][i]; lane gets W[tok][4 consecutive ch]
      constexpr int NTI = (CH / 16) * (DK / 16);
      for (int t = w; t < NTI; t += 8) {
        const int mt = t % (CH / 16), nt = t / (CH / 16);
        f32x4 acc = zero4();
        if constexpr (BWD)
          acc = tile_mm_ps<OP, CH>(sKpT, L::LDT, 16 * nt, sTe, sTeL, L::LDT, 16 * mt);
        else
          acc = tile_mm<CH>([&](int rr, int k) { return frag_row<OP>(sKpT, L::LDT, 16 * nt + rr, k); },
                            [&](int rr, int k) { return frag_row<OP>(sTe, L::LDT, 16 * mt + rr, k); }, acc);
        store4<OP>(wW + (16 * mt + r16) * DK + 16 * nt + 4 * q4, acc[0], acc[1], acc[2], acc[3]);
      }
      // U~ tiles: C[tok][dv]; lane holds 4 consecutive tokens of one value column -> U~^T rows
      // (fp32 for the backward, where its rounding would reach the gradients)
      constexpr int NTU = (CH / 16) * (DV / 16);
      for (int t = w; t < NTU; t += 8) {
        const int mt = t % (CH / 16), nt = t / (CH / 16);
        f32x4 acc = zero4();
        if constexpr (BWD) {
#pragma unroll
          for (int k = 0; k < CH; k += 32)
            acc = mma_sp(sfrag_pair<OP>(sTe, sTeL, L::LDT, 16 * mt + r16, k + 8 * q4),
                         frag_row<OP>(sVT, L::LDT, 16 * nt + r16, k + 8 * q4), acc);
        } else {
          acc = tile_mm<CH>([&](int rr, int k) { return frag_row<OP>(sTe, L::LDT, 16 * mt + rr, k); },
                            [&](int rr, int k) { return frag_row<OP>(sVT, L::LDT, 16 * nt + rr, k); }, acc);
        }
        if constexpr (BWD)
          *reinterpret_cast<f32x4*>(a.wsUtF + blk * WB::UTF + (16 * nt + r16) * CH + 16 * mt + 4 * q4) = acc;
        else
          store4<OP>(reinterpret_cast<OP*>(a.wsUt) + blk * WB::UT + (16 * nt + r16) * CH + 16 * mt + 4 * q4, acc[0],
                     acc[1], acc[2], acc[3]);
      }
    }
    }   // !skip
    item = nitem;
    ci = nci;
    nitem = n2item;
    nrec = n2rec;
  }
}

// ---------------------------------------------------------------------------
// sequential state pass (forward outputs, or the per-chunk states for backward)
// ---------------------------------------------------------------------------
// One work-group walks the chunks of one (sequence, head, value slice of DVS
// columns) in order.  Eight waves: waves 0-3 form U = U~ - W S for token tile
// w, waves 4-7 form Qt S and then the output rows of tile w-4; every wave
// updates its 16x16 tiles of S.  S stays in fp32 registers; each chunk it is
// copied to LDS in the operand type for the products that read it.  The next
// chunk's matrices are loaded into registers while the current one computes.
// UF: U~ is read in fp32 (the copy a training-mode prep writes) rather than in
// the operand type.  With UF and 2-byte operands (KS) the state update takes Kh
// and U as split (hi, lo) pairs: the backward's dlog alpha collects the rounding
// of every saved state (through dGamma_C), and plain fp16 Kh and U would put
// about 2^-11 of each chunk's update into it.  The training prep writes Kh^T's
// lo half beside the hi half (wsKhTL).
template <typename E, int DK, int DV, int DVS, bool OUT, bool SAVE, bool UF = SAVE>
struct StateLds {
  using OP = typename OpOf<E>::T;
  static constexpr bool KS = UF && sizeof(OP) == 2;
  static constexpr int P = PADE<OP>;
  static constexpr int LDK = DK + P;
  static constexpr int LDT = CH + P;
  static constexpr size_t W = 0;                                                  // OP [CH][LDK]
  static constexpr size_t QT = W + (size_t)CH * LDK * sizeof(OP);                 // OP [CH][LDK]  (OUT)
  static constexpr size_t KHT = QT + (OUT ? (size_t)CH * LDK * sizeof(OP) : 0);   // OP [DK][LDT]
  static constexpr size_t AQK = KHT + (size_t)DK * LDT * sizeof(OP);              // OP [CH][LDT]  (OUT)
  using UTT = typename std::conditional<UF, float, OP>::type;                    // U~ element type
  static constexpr size_t UT = AQK + (OUT ? (size_t)CH * LDT * sizeof(OP) : 0);   // UTT [DVS][CH]
  static constexpr size_t GAM = UT + (size_t)DVS * CH * sizeof(UTT);              // float [DK]
  static constexpr size_t ST = GAM + (size_t)DK * 4;                              // OP [DVS][LDK]  S^T
  static constexpr size_t UL = ST + (size_t)DVS * LDK * sizeof(OP);               // OP [DVS][LDT]  U^T
  static constexpr size_t KHL = UL + (size_t)DVS * LDT * sizeof(OP);              // OP [DK][LDT]   Kh^T lo (KS)
  static constexpr size_t ULL = KHL + (KS ? (size_t)DK * LDT * sizeof(OP) : 0);   // OP [DVS][LDT]  U^T lo (KS)
  static constexpr size_t BYTES = ULL + (KS ? (size_t)DVS * LDT * sizeof(OP) : 0);
  static_assert(BYTES <= 163840, "state LDS");
};

// PF = 2: operands of chunk n+2 are in flight while chunk n+1 waits in
// registers (one work-group per CU); PF = 1: one set of staging registers, so
// the kernel fits 4 waves per SIMD and two work-groups share a CU.
// MODE 1: the transfer of a stretch of chunks instead of a state.  The chunk
// step S' = Gamma_C S + Kh^T (U~ - W S) is affine in S; run from S = I with
// U~ = 0 it gives M = prod_n (Diag(Gamma_C) - Kh_n^T W_n) (dk x dk, DV = DK),
// and S_end = M S_start + (the same run from S = 0 with U~).  MODE 2: one
// launch of both, the first half of the grid the runs from S = 0 (end states
// to final_state), the second half the transfers (to seg_m).
template <typename E, typename O, int DK, int DV, int DVS, bool OUT, bool SAVE, int PF, int MODE = 0, bool UF = SAVE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(PF == 1 ? 4 : 1, PF == 1 ? 4 : 2))) void kda_state(const Args a) {
  static_assert(MODE == 0 || (!OUT && !SAVE && DV == DK), "transfer runs keep only the end state");
  const bool xf = MODE == 1 || (MODE == 2 && blockIdx.x >= gridDim.x / 2);
  const int bid = (MODE == 2 && xf) ? (int)(blockIdx.x - gridDim.x / 2) : (int)blockIdx.x;
  using L = StateLds<E, DK, DV, DVS, OUT, SAVE, UF>;
  using OP = typename L::OP;
  using WB = WsBlock<E, DK, DV>;
  constexpr int NT = 512, NSL = DV / DVS;
  constexpr int MTS = DK / 16, NTS = DVS / 16;   // state tiles (channel x column)
  constexpr int NST = MTS * NTS;
  constexpr int SPW = (NST + 7) / 8;             // state tiles per wave (tile t -> wave t % 8)
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

  int unit, sl;
  if (!xcd_unit(bid, NSL, a.N * a.H, unit, sl)) return;
  const int seq = a.seq_order[unit / a.H], h = unit % a.H, H = a.H;   // longest sequences first
  const int n0 = sl * DVS;
  const int l = lane_id(), w = wave_id(), r16 = l & 15, q4 = l >> 4;
  __builtin_assume(w < 8);   // 512 threads: every state tile t = w + 8 i < NST is then known in range
  const int c0 = a.seq_chunk0[seq], nch = a.seq_chunk0[seq + 1] - c0;
  // token range of the sequence, from its first and last chunk (read once, so
  // the only global loads inside the loop are the prefetch of the next chunk)
  int tbeg = 0, tend = 0;
  if (nch > 0) {
    const ChunkInfo first = a.chunks[c0], last = a.chunks[c0 + nch - 1];
    tbeg = first.t0;
    tend = last.t0 + last.len;
  }

  OP* sW = reinterpret_cast<OP*>(smem + L::W);
  OP* sQt = reinterpret_cast<OP*>(smem + L::QT);
  OP* sKhT = reinterpret_cast<OP*>(smem + L::KHT);
  OP* sAqk = reinterpret_cast<OP*>(smem + L::AQK);
  using UTT = typename L::UTT;
  UTT* sUt = reinterpret_cast<UTT*>(smem + L::UT);
  float* sGam = reinterpret_cast<float*>(smem + L::GAM);
  OP* sST = reinterpret_cast<OP*>(smem + L::ST);
  OP* sUL = reinterpret_cast<OP*>(smem + L::UL);
  constexpr bool KS = L::KS;
  OP* sKhL = reinterpret_cast<OP*>(smem + L::KHL);
  OP* sULL = reinterpret_cast<OP*>(smem + L::ULL);

  // kernel-argument fields are copied to locals so the argument block never
  // has its address taken (that would place it in scratch)
  const OP* gW = reinterpret_cast<const OP*>(a.wsW);
  const OP* gQt = reinterpret_cast<const OP*>(a.wsQt);
  const OP* gAqk = reinterpret_cast<const OP*>(a.wsAqk);
  const OP* gKhT = reinterpret_cast<const OP*>(a.wsKhT);
  const OP* gKhTL = reinterpret_cast<const OP*>(a.wsKhTL);   // KS: Kh^T lo, same blocks as Kh^T
  const UTT* gUt = UF ? reinterpret_cast<const UTT*>(a.wsUtF) : reinterpret_cast<const UTT*>(a.wsUt);
  const float* gGam = a.wsGam;
  float* gS = reinterpret_cast<float*>(a.wsS);
  float* gU = a.wsU;
  O* gOut = reinterpret_cast<O*>(a.out);
  const float scale = a.scale;
  const float* gInit = a.init;
  float* gFinal = (MODE == 2 && xf) ? a.seg_m : a.final_state;

  f32x4 S[SPW];
  const size_t st_off = ((size_t)seq * H + h) * DK * DV;
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int t = w + 8 * i, mt = t % MTS, nt = t / MTS;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int ch = 16 * mt + 4 * q4 + ii, col = n0 + 16 * nt + r16;
      if (xf)
        S[i][ii] = (t < NST && ch == col) ? 1.f : 0.f;
      else
        S[i][ii] = (gInit && t < NST) ? gInit[st_off + (size_t)ch * DV + col] : 0.f;
    }
  }

  // Staging registers: chunk n + PF is loaded while chunk n is in LDS.  With PF = 2
  // (a build option) a second set lets chunk n + 2 be in flight while chunk n + 1
  // waits in registers; the default PF = 1 measures as fast.  Separate objects of a
  // native vector type stay in VGPRs.
  struct Stage {
    TileCopy<OP, CH, DK, NT> w;
    TileCopy<OP, (OUT ? CH : 1), (OUT ? DK : 16 / sizeof(OP)), NT> qt;
    TileCopy<OP, DK, CH, NT> kht;
    TileCopy<OP, (KS ? DK : 1), (KS ? CH : 16 / sizeof(OP)), NT> khtl;   // Kh^T lo (KS)
    TileCopy<OP, (OUT ? CH : 1), (OUT ? CH : 16 / sizeof(OP)), NT> aqk;
    TileCopy<UTT, DVS, CH, NT> ut;
    TileCopy<float, 1, DK, NT> gam;
  };
  Stage st0;
  [[maybe_unused]] Stage st1;
  auto blk_of = [&](int n) { return (size_t)(c0 + n) * H + h; };
  // a chunk's operands -> registers, in two parts issued at different points of a step
  // (the memory queue then never holds all of them ahead of the step's stores)
  auto stage_load_a = [&](Stage& p, int n) __attribute__((always_inline)) {
    const size_t b = blk_of(n);
    p.kht.load(gKhT + b * WB::KHT, CH);
    if constexpr (KS) p.khtl.load(gKhTL + b * WB::KHT, CH);
  };
  auto stage_load = [&](Stage& p, int n) __attribute__((always_inline)) {
    const size_t b = blk_of(n);
    p.w.load(gW + b * WB::W, DK);
    if constexpr (OUT) {
      p.qt.load(gQt + b * WB::QT, DK);
      p.aqk.load(gAqk + b * WB::AQK, CH);
    }
    if (!xf) p.ut.load(gUt + b * WB::UT + (size_t)n0 * CH, CH);  // UT == UTF element count
    p.gam.load(gGam + b * WB::GAM, DK);
  };
  auto stage_store = [&](const Stage& p) __attribute__((always_inline)) {
    p.w.store(sW, L::LDK);
    if constexpr (OUT) {
      p.qt.store(sQt, L::LDK);
      p.aqk.store(sAqk, L::LDT);
    }
    p.kht.store(sKhT, L::LDT);
    if constexpr (KS) p.khtl.store(sKhL, L::LDT);
    if (!xf) p.ut.store(sUt, CH);
    p.gam.store(sGam, DK);
  };

  const size_t ro = (size_t)H * DV;
  // one chunk: LDS holds chunk n; `ld` receives chunk n+PF (clamped, so its
  // registers are always defined); `nx` holds chunk n+1 and goes to LDS at the end
  auto chunk = [&](int n, Stage& ld, const Stage& nx) __attribute__((always_inline)) {
    // S -> LDS in the operand type, transposed ([column][channel])
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = w + 8 * i, mt = t % MTS, nt = t / MTS;
      if (t < NST) {
        store4<OP>(sST + (16 * nt + r16) * L::LDK + 16 * mt + 4 * q4, S[i][0], S[i][1], S[i][2], S[i][3]);
        if constexpr (SAVE) {
          // backward needs the state entering every chunk: fp32 [DK][DV] per chunk-head; after
          // a quad transpose a lane stores 4 columns of row 16 mt + 4 q4 + (r16 & 3)
          const int g4 = r16 & ~3, ri = r16 & 3;
          *reinterpret_cast<f32x4*>(gS + blk_of(n) * WB::S + (size_t)(16 * mt + 4 * q4 + ri) * DV + n0 + 16 * nt + g4) =
              quad_transpose(S[i]);
        }
      }
    }
    __syncthreads();
    stage_load_a(ld, min(n + PF, nch - 1));   // first part, after this step's S stores

    f32x4 o1[NTS];
    if (w < 4) {
      // X = W S (token tile w); U = U~ - X -> LDS ([column][token])
#pragma unroll
      for (int nt = 0; nt < NTS; ++nt) {
        const f32x4 x = tile_mm<DK>([&](int rr, int k) { return frag_row<OP>(sW, L::LDK, 16 * w + rr, k); },
                                    [&](int rr, int k) { return frag_row<OP>(sST, L::LDK, 16 * nt + rr, k); },
                                    zero4());
        float ut[4] = {0.f, 0.f, 0.f, 0.f};
        if (!xf) load4<UTT>(sUt + (16 * nt + r16) * CH + 16 * w + 4 * q4, ut);
        const int uo = (16 * nt + r16) * L::LDT + 16 * w + 4 * q4;
        if constexpr (KS)
          store4_split<OP>(sUL + uo, sULL + uo, ut[0] - x[0], ut[1] - x[1], ut[2] - x[2], ut[3] - x[3]);
        else
          store4<OP>(sUL + uo, ut[0] - x[0], ut[1] - x[1], ut[2] - x[2], ut[3] - x[3]);
        if constexpr (SAVE) {
          // and U in fp32, token-major [CH][DV] (quad transpose, as S above)
          const int g4 = r16 & ~3, ri = r16 & 3;
          *reinterpret_cast<f32x4*>(gU + blk_of(n) * WB::U + (size_t)(16 * w + 4 * q4 + ri) * DV + n0 + 16 * nt + g4) =
              quad_transpose(f32x4{ut[0] - x[0], ut[1] - x[1], ut[2] - x[2], ut[3] - x[3]});
        }
      }
    } else if constexpr (OUT) {
#pragma unroll
      for (int nt = 0; nt < NTS; ++nt)
        o1[nt] = tile_mm<DK>([&](int rr, int k) { return frag_row<OP>(sQt, L::LDK, 16 * (w - 4) + rr, k); },
                             [&](int rr, int k) { return frag_row<OP>(sST, L::LDK, 16 * nt + rr, k); }, zero4());
    }
    __syncthreads();
    // second part, after this step's U stores: stores issued behind the loads would wait
    // for them in the memory queue
    stage_load(ld, min(n + PF, nch - 1));

    if constexpr (OUT) {
      if (w >= 4) {
        const int tt = w - 4;
        const int t0 = tbeg + n * CH, clen = min(CH, tend - t0);
        O* oh = gOut + (size_t)t0 * ro + (size_t)h * DV + n0;
        // all tiles' products first, then one guarded group of stores: a guard per tile
        // would end a basic block after each tile and serialise their latencies
        f32x4 y[NTS];
#pragma unroll
        for (int nt = 0; nt < NTS; ++nt)
          y[nt] = tile_mm<CH>([&](int rr, int k) { return frag_row<OP>(sAqk, L::LDT, 16 * tt + rr, k); },
                              [&](int rr, int k) { return frag_row<OP>(sUL, L::LDT, 16 * nt + rr, k); }, o1[nt]);
        // quad transpose: this lane stores 4 columns of token 16 tt + 4 q4 + (r16 & 3)
#pragma unroll
        for (int nt = 0; nt < NTS; ++nt) y[nt] = quad_transpose(scale * y[nt]);
        const int tok = 16 * tt + 4 * q4 + (r16 & 3);
        if (tok < clen) {
#pragma unroll
          for (int nt = 0; nt < NTS; ++nt)
            store4<O>(oh + (size_t)tok * ro + 16 * nt + (r16 & ~3), y[nt][0], y[nt][1], y[nt][2], y[nt][3]);
        }
      }
    }
    // S' = Gamma_C * S + Kh^T U
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = w + 8 * i, mt = t % MTS, nt = t / MTS;
      if (t < NST) {
        f32x4 x = zero4();
        if constexpr (KS) {
#pragma unroll
          for (int k = 0; k < CH; k += 32)
            x = mma_ss(sfrag_pair<OP>(sKhT, sKhL, L::LDT, 16 * mt + r16, k + 8 * q4),
                       sfrag_pair<OP>(sUL, sULL, L::LDT, 16 * nt + r16, k + 8 * q4), x);
        } else {
          x = tile_mm<CH>([&](int rr, int k) { return frag_row<OP>(sKhT, L::LDT, 16 * mt + rr, k); },
                          [&](int rr, int k) { return frag_row<OP>(sUL, L::LDT, 16 * nt + rr, k); }, x);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) S[i][ii] = sGam[16 * mt + 4 * q4 + ii] * S[i][ii] + x[ii];
      }
    }
    __syncthreads();
    if (n + 1 < nch) stage_store(nx);
  };

  if (nch > 0) {
    stage_load_a(st0, 0);
    stage_load(st0, 0);
    stage_store(st0);
    if constexpr (PF == 2) {
      stage_load_a(st1, min(1, nch - 1));
      stage_load(st1, min(1, nch - 1));
    }
  }
  if constexpr (PF == 2) {
    for (int n = 0; n < nch; n += 2) {
      chunk(n, st0, st1);
      if (n + 1 < nch) chunk(n + 1, st1, st0);
    }
  } else {
    for (int n = 0; n < nch; ++n) chunk(n, st0, st0);
  }

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

// Compute units of the current device (the persistent prep runs one work-group on each).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Value columns per work-group of a sequential pass (bf16 inputs): the widest
// slice that still gives every compute unit a work-group.  Wider slices stage the
// per-chunk operands for more columns at once; a grid shorter than the CU count
// leaves CUs idle while the longest chain runs.
int pick_dvs(int units, int dv) {
#ifdef KDA_FORCE_DVS
  (void)units;
  (void)dv;
  return KDA_FORCE_DVS;
#else
  return (dv >= 64 && (long long)units * (dv / 64) >= device_cus()) ? 64 : 16;
#endif
}

template <typename E, typename O, int DK, int DV, int DVS, bool OUT, bool SAVE, int MODE = 0, bool UF = SAVE>
static hipError_t launch_state(const Args& a, hipStream_t st, const char* name = nullptr) {
  constexpr int NSL = DV / DVS;
  const int units = a.N * a.H;
  const int groups = (units + 7) / 8;
  const int grid = groups * 8 * NSL * (MODE == 2 ? 2 : 1);
  if (grid == 0) return hipSuccess;
  constexpr int PF = KDA_STATE_PF;
  if (!name) name = OUT ? (SAVE ? "kda_state_fwd_save" : "kda_state_fwd") : "kda_state_bwd_fwdpass";
  KDA_TIMED(name, st,
            hipLaunchKernelGGL((kda_state<E, O, DK, DV, DVS, OUT, SAVE, PF, MODE, UF>), dim3(grid), dim3(512), 0, st, a));
  return hipGetLastError();
}

template <typename E, typename O, int DK, int DV, bool OUT, bool SAVE, int MODE = 0, bool UF = SAVE>
static hipError_t launch_state_auto(const Args& a, hipStream_t st, const char* name = nullptr) {
  const int units = a.N * a.H * (MODE == 2 ? 2 : 1);
  if constexpr (sizeof(E) == 2) {
    if (pick_dvs(units, DV) == 64) return launch_state<E, O, DK, DV, 64, OUT, SAVE, MODE, UF>(a, st, name);
    return launch_state<E, O, DK, DV, 16, OUT, SAVE, MODE, UF>(a, st, name);
  } else {
    return launch_state<E, O, DK, DV, 32, OUT, SAVE, MODE, UF>(a, st, name);
  }
}

// ---------------------------------------------------------------------------
// segment scan (the single-GPU half of splitting one long sequence over
// ranks): each sequence is cut into `segs` stretches of whole chunks.  Every
// stretch runs in parallel twice: from S = 0 with U~ (its end state S_loc)
// and as a transfer M from S = I without U~.  A short sequential scan per
// (sequence, head) then gives each stretch its entering state,
// S_in(p + 1) = M(p) S_in(p) + S_loc(p), and the ordinary state pass runs all
// stretches at once from those states, writing the outputs.
// ---------------------------------------------------------------------------
int fwd_segments(int N, int H, int dv, long long tokens, bool save) {
  if (const char* env = std::getenv("KDA_SEGMENTS")) {   // explicit stretch count (tests, tuning)
    const int p = std::atoi(env);
    if (p >= 1) return std::min(p, 64);
  }
  (void)save;   // training mode segments the same way (the backward reuses the transfers)
  if (N <= 0) return 1;
  // enough stretches that 64-column slices give every CU a chain (measured on
  // one 128K-token sequence with 16 heads: 8 stretches 3.8 ms, 4 stretches
  // 4.8 ms, none 5.4 ms; more than 8 lose to the longer scan)
  const long long units = (long long)N * H * std::max(1, dv / 64);
  const long long avg_chunks = tokens / CH / N;
  if (units >= device_cus() || avg_chunks < 256) return 1;
  long long p = (device_cus() + units - 1) / units;
  p = std::min<long long>(p, std::min<long long>(8, avg_chunks / 64));
  return (int)std::max<long long>(p, 1);
}

__global__ __launch_bounds__(256) void kda_segment_map(const int32_t* __restrict__ sc0, int N, int P,
                                                      int32_t* __restrict__ vsc0, int32_t* __restrict__ vord) {
  for (int v = blockIdx.x * blockDim.x + threadIdx.x; v <= N * P; v += gridDim.x * blockDim.x) {
    if (v == N * P) {
      vsc0[v] = sc0[N];
    } else {
      const int n = v / P, p = v % P;
      const int c0 = sc0[n], nch = sc0[n + 1] - c0;
      vsc0[v] = c0 + (int)((long long)nch * p / P);
      vord[v] = v;
    }
  }
}

// One work-group per (sequence, head): S (fp32, [DK][DV]) and the stretch's
// transfer M ([DK][DK]) in LDS; each wave owns 16x16 tiles of the new state and
// forms them with fp32 MFMA (16 channels of the contraction per step, in order:
// bitwise reproducible).
template <int DK, int DV>
__global__ __launch_bounds__(512) void kda_segment_scan(const Args a) {
  constexpr int LS = DV + 4, LM = DK + 4;   // padded rows
  __shared__ __attribute__((aligned(16))) float sS[DK * LS];
  __shared__ __attribute__((aligned(16))) float sM[DK * LM];
  constexpr int NT = 512, NTILE = (DK / 16) * (DV / 16), TPW = (NTILE + 7) / 8;
  const int n = blockIdx.x / a.H, h = blockIdx.x % a.H, P = a.segs, tid = threadIdx.x;
  const int w = wave_id(), l = lane_id(), r16 = l & 15, q4 = l >> 4;
  constexpr size_t SZ = (size_t)DK * DV, MZ = (size_t)DK * DK;
  const float* init = a.init ? a.init + ((size_t)n * a.H + h) * SZ : nullptr;
  for (int o = tid; o < DK * DV; o += NT) sS[(o / DV) * LS + o % DV] = init ? init[o] : 0.f;
  __syncthreads();
  for (int p = 0; p < P; ++p) {
    const size_t v = ((size_t)n * P + p) * a.H + h;
    for (int o = tid; o < DK * DV; o += NT) a.seg_in[v * SZ + o] = sS[(o / DV) * LS + o % DV];
    for (int o = tid; o < DK * DK; o += NT) sM[(o / DK) * LM + o % DK] = a.seg_m[v * MZ + o];
    __syncthreads();
    f32x4 acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = w + 8 * i, mt = t % (DK / 16), nt = t / (DK / 16);
      acc[i] = zero4();
      if (t < NTILE) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          acc[i][ii] = a.seg_loc[v * SZ + (size_t)(16 * mt + 4 * q4 + ii) * DV + 16 * nt + r16];
        for (int kb = 0; kb < DK / 16; ++kb)
          acc[i] = mm16_f32(sM + 16 * mt * LM + 16 * kb, LM, sS + 16 * kb * LS + 16 * nt, LS, acc[i]);
      }
    }
    __syncthreads();   // every read of this stretch's S and M is done
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = w + 8 * i, mt = t % (DK / 16), nt = t / (DK / 16);
      if (t < NTILE) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sS[(16 * mt + 4 * q4 + ii) * LS + 16 * nt + r16] = acc[i][ii];
      }
    }
    __syncthreads();
  }
  if (a.final_state)
    for (int o = tid; o < DK * DV; o += NT) a.final_state[((size_t)n * a.H + h) * SZ + o] = sS[(o / DV) * LS + o % DV];
}

// Reverse scan for the backward (the transposed maps): the gradient of the
// state entering stretch p is dS_in(p) = M(p)^T dS_out(p) + dS_loc(p), where
// dS_loc(p) is stretch p's reverse pass run from zero and dS_out(p) =
// dS_in(p + 1) (dS_final for the last stretch).  Writes dS_out(p) of every
// stretch to seg_in and d_init_state = dS_in(0).  One work-group per
// (sequence, head); M^T is staged in LDS and the products are fp32 MFMA in a
// fixed order.
template <int DK, int DV>
__global__ __launch_bounds__(512) void kda_segment_rscan(const Args a) {
  constexpr int LS = DV + 4, LM = DK + 4;   // padded rows
  __shared__ __attribute__((aligned(16))) float sS[DK * LS];
  __shared__ __attribute__((aligned(16))) float sM[DK * LM];   // M^T
  constexpr int NT = 512, NTILE = (DK / 16) * (DV / 16), TPW = (NTILE + 7) / 8;
  const int n = blockIdx.x / a.H, h = blockIdx.x % a.H, P = a.segs, tid = threadIdx.x;
  const int w = wave_id(), l = lane_id(), r16 = l & 15, q4 = l >> 4;
  constexpr size_t SZ = (size_t)DK * DV, MZ = (size_t)DK * DK;
  const float* dfin = a.dfinal ? a.dfinal + ((size_t)n * a.H + h) * SZ : nullptr;
  // the scan runs on scaled gradients (the stretches' local runs read dO times s);
  // d_init_state is stored unscaled
  const float gs = a.gscale ? a.gscale[0] : 1.f, gs_inv = a.gscale ? a.gscale[1] : 1.f;
  for (int o = tid; o < DK * DV; o += NT) sS[(o / DV) * LS + o % DV] = dfin ? gs * dfin[o] : 0.f;
  __syncthreads();
  for (int p = P - 1; p >= 0; --p) {
    const size_t v = ((size_t)n * P + p) * a.H + h;
    for (int o = tid; o < DK * DV; o += NT) a.seg_in[v * SZ + o] = sS[(o / DV) * LS + o % DV];
    for (int o = tid; o < DK * DK; o += NT) sM[(o % DK) * LM + o / DK] = a.seg_m[v * MZ + o];
    __syncthreads();
    f32x4 acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = w + 8 * i, mt = t % (DK / 16), nt = t / (DK / 16);
      acc[i] = zero4();
      if (t < NTILE) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          acc[i][ii] = a.seg_loc[v * SZ + (size_t)(16 * mt + 4 * q4 + ii) * DV + 16 * nt + r16];
        for (int kb = 0; kb < DK / 16; ++kb)
          acc[i] = mm16_f32(sM + 16 * mt * LM + 16 * kb, LM, sS + 16 * kb * LS + 16 * nt, LS, acc[i]);
      }
    }
    __syncthreads();   // every read of this stretch's dS and M^T is done
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = w + 8 * i, mt = t % (DK / 16), nt = t / (DK / 16);
      if (t < NTILE) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sS[(16 * mt + 4 * q4 + ii) * LS + 16 * nt + r16] = acc[i][ii];
      }
    }
    __syncthreads();
  }
  if (a.dinit)
    for (int o = tid; o < DK * DV; o += NT) a.dinit[((size_t)n * a.H + h) * SZ + o] = gs_inv * sS[(o / DV) * LS + o % DV];
}

hipError_t launch_segment_map(const Args& a, hipStream_t st) {
  const int NV = a.N * a.segs;
  KDA_TIMED("kda_seg_map", st,
            hipLaunchKernelGGL(kda_segment_map, dim3((NV + 256) / 256), dim3(256), 0, st, a.seq_chunk0, a.N, a.segs,
                               a.vsc0, a.vord));
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_segment_rscan(const Args& a, hipStream_t st) {
  KDA_TIMED("kda_seg_rscan", st,
            hipLaunchKernelGGL((kda_segment_rscan<DK, DV>), dim3(a.N * a.H), dim3(512), 0, st, a));
  return hipGetLastError();
}
template hipError_t launch_segment_rscan<64, 64>(const Args&, hipStream_t);
template hipError_t launch_segment_rscan<64, 128>(const Args&, hipStream_t);
template hipError_t launch_segment_rscan<128, 64>(const Args&, hipStream_t);
template hipError_t launch_segment_rscan<128, 128>(const Args&, hipStream_t);

// TRAIN: the prep ran in training mode (fp32 U~) and the final pass keeps the
// backward's intermediates; OUT: the final pass writes the outputs.
template <typename E, typename O, int DK, int DV, bool TRAIN, bool OUT>
static hipError_t launch_segmented_state(const Args& a, hipStream_t st) {
  const int P = a.segs, NV = a.N * P;
  hipError_t e = launch_segment_map(a, st);
  if (e != hipSuccess) return e;
  Args av = a;   // the stretches as sequences of their own
  av.N = NV;
  av.seq_chunk0 = a.vsc0;
  av.seq_order = a.vord;
  av.out = nullptr;
  Args al = av;   // end state of each stretch from zero, and (same launch when dk == dv) its transfer
  al.init = nullptr;
  al.final_state = a.seg_loc;
  if constexpr (DK == DV) {
    if ((e = launch_state_auto<E, O, DK, DV, false, false, 2, TRAIN>(al, st, "kda_seg_local_transfer")) != hipSuccess)
      return e;
  } else {
    if ((e = launch_state_auto<E, O, DK, DV, false, false, 0, TRAIN>(al, st, "kda_seg_local")) != hipSuccess) return e;
    Args am = av;
    am.init = nullptr;
    am.final_state = a.seg_m;
    if ((e = launch_state_auto<E, O, DK, DK, false, false, 1, TRAIN>(am, st, "kda_seg_transfer")) != hipSuccess)
      return e;
  }
  KDA_TIMED("kda_seg_scan", st,
            hipLaunchKernelGGL((kda_segment_scan<DK, DV>), dim3(a.N * a.H), dim3(512), 0, st, a));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  Args ab = av;   // every stretch from its true entering state, with the outputs (and what the backward keeps)
  ab.out = a.out;
  ab.init = a.seg_in;
  ab.final_state = nullptr;
  return launch_state_auto<E, O, DK, DV, OUT, TRAIN>(ab, st);
}

// BWD: also keep what the backward pass needs (T, the un-beta Gram, fp32 Kh and U~).
template <typename E, int DK, int DV, bool BWD>
static hipError_t launch_prep(const Args& a, hipStream_t st, const char* name) {
  if (a.max_chunks == 0 || a.H == 0) return hipSuccess;
  if constexpr (sizeof(E) == 2) {
    const long long items = (long long)a.max_chunks * a.H;
    const int grid = (int)std::min<long long>(items, device_cus());
#define KDA_PREP8(QKN, GATE)                                                                                \
  do {                                                                                                       \
    KDA_TIMED(name, st, hipLaunchKernelGGL((kda_prep8<DK, DV, BWD, QKN, GATE, 0>), dim3(grid), dim3(512), 0, st, a)); \
    KDA_TIMED("kda_prep_steep", st,                                                                          \
              hipLaunchKernelGGL((kda_prep8<DK, DV, BWD, QKN, GATE, 1>), dim3(grid), dim3(512), 0, st, a));  \
  } while (0)
    if (a.qk_norm && a.gate_ls)
      KDA_PREP8(true, true);
    else if (a.qk_norm)
      KDA_PREP8(true, false);
    else if (a.gate_ls)
      KDA_PREP8(false, true);
    else
      KDA_PREP8(false, false);
#undef KDA_PREP8
  } else {
    if (a.qk_norm)
      KDA_TIMED(name, st,
                hipLaunchKernelGGL((kda_prep<E, DK, DV, BWD, true>), dim3(a.max_chunks, a.H), dim3(256), 0, st, a));
    else
      KDA_TIMED(name, st,
                hipLaunchKernelGGL((kda_prep<E, DK, DV, BWD, false>), dim3(a.max_chunks, a.H), dim3(256), 0, st, a));
  }
  return hipGetLastError();
}

// Forward pass; with `save` it also leaves in the workspace everything the
// backward pass would otherwise recompute (T, G, fp32 Kh and U~, S entering
// every chunk, U), so a following kda_bwd on the same workspace skips that work.
template <typename E, typename O, int DK, int DV>
hipError_t launch_fwd(const Args& a, hipStream_t st, bool save) {
  hipError_t e = launch_chunk_map(a, st);
  if (e != hipSuccess) return e;
  if (save) {
    if constexpr (sizeof(E) == 4 && DK == 128) {
      return hipErrorInvalidValue;   // no fp32 backward at dk = 128, so nothing to save for
    } else {
      e = launch_prep<E, DK, DV, true>(a, st, "kda_prep_save");
      if (e != hipSuccess) return e;
      if (a.segs > 1) return launch_segmented_state<E, O, DK, DV, true, true>(a, st);
      return launch_state_auto<E, O, DK, DV, true, true>(a, st);
    }
  }
  e = launch_prep<E, DK, DV, false>(a, st, "kda_prep");
  if (e != hipSuccess) return e;
  if (a.segs > 1) return launch_segmented_state<E, O, DK, DV, false, true>(a, st);
  return launch_state_auto<E, O, DK, DV, true, false>(a, st);
}

// front half of the backward pass: chunk map, chunk-local prep (also keeping
// T), and the states entering every chunk
template <typename E, int DK, int DV>
hipError_t launch_bwd_front(const Args& a, hipStream_t st) {
  hipError_t e = launch_chunk_map(a, st);
  if (e != hipSuccess) return e;
  e = launch_prep<E, DK, DV, true>(a, st, "kda_prep_bwd");
  if (e != hipSuccess) return e;
  if (a.segs > 1) return launch_segmented_state<E, float, DK, DV, true, false>(a, st);
  return launch_state_auto<E, float, DK, DV, false, true>(a, st);
}

#define KDA_INST(E, DK, DV)                                                                   \
  template hipError_t launch_fwd<E, float, DK, DV>(const Args&, hipStream_t, bool);           \
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
#define KDA_INST_BF16OUT(DK, DV) template hipError_t launch_fwd<bf16, bf16, DK, DV>(const Args&, hipStream_t, bool);
KDA_INST_BF16OUT(64, 64)
KDA_INST_BF16OUT(64, 128)
KDA_INST_BF16OUT(128, 64)
KDA_INST_BF16OUT(128, 128)
#undef KDA_INST_BF16OUT

}  // namespace kda
