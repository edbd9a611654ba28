// kda_bwd.hip -- backward pass of Kimi Delta Attention on gfx950.
//
// Reverse-mode differentiation of the chunked forward (see kda_fwd.hip), for
// L = <d_out, o> + <d_final_state, S_T>.  Per chunk, with S the state entering
// it, dS' the gradient of the state leaving it and dO the output gradient:
//
//   dU   = scale Aqk^T dO + Kh dS'                  dS = Gamma_C dS' + scale Qt^T dO - W^T dU
//   dAqk = scale tril(dO U^T)    dQt = scale dO S^T + dAqk K-    dK- = dAqk^T Qt
//   dKh  = U dS'^T               dGamma_C = rowsum(dS' * S)      dW = -dU S^T
//   dT   = dW (b K+)^T + dU (b V)^T       dK+ = b T^T dW,  dV = b T^T dU
//   dA   = -strict_tril(T^T dT T^T)       dG = diag(b) dA  (A = diag(b) G)
//   dK+ += dG K-,   dK- += dG^T K+,   dbeta = rowsums of K+ T^T dW, V T^T dU, dA G
//   dg   = dK+ K+ - dK- K- + dQt Qt - dKh Kh,   dg_C += sum_r dKh Kh + dGamma_C Gamma_C
//   dlog_alpha = reverse cumulative sum of dg over the chunk
//
// Launch sequence (the front half is shared with the forward, kda_fwd.hip):
//   chunk map, prep (also T, G, fp32 Kh), state pass (S entering each chunk, U),
//   kda_state_rev   : reverse sequential pass over the chunks of one (sequence,
//                     head, value slice): dS', dU and d_init_state.
//   kda_bwd_chunk   : chunk-parallel; contractions over the value dimension,
//                     then over tokens, the gated products, and the assembly
//                     of dq, dk, dv, dlog_alpha, dbeta.
// The gated products never form K- = K/Gamma: they use the same per-block
// reference rows as the forward's decayed Gram blocks.
#include "kda_internal.hpp"

namespace kda {

template <typename E, int DK, int DV>
hipError_t launch_bwd_front(const Args& a, hipStream_t st);

// ---------------------------------------------------------------------------
// scale of the upstream gradients (bf16 inputs)
// ---------------------------------------------------------------------------
// The bf16 backward narrows dO, dS' and dU to fp16 (hi, lo) pairs, whose range
// (normal from 6.1e-5 up to 65504) is far narrower than bf16's.  The backward is
// linear in (dO, dS_final), so the kernels run on s dO and s dS_final, with s the
// power of two that puts the largest magnitude of both in [0.5, 1), and multiply
// every gradient they store by 1/s; both scalings are exact.  s = 1 when the
// maximum is 0, inf or NaN (the non-finite values then reach the gradients as
// they would without the scale).
__global__ __launch_bounds__(256) void kda_grad_absmax(const bf16* __restrict__ dout, size_t n_out,
                                                       const float* __restrict__ dfin, size_t n_fin,
                                                       float* __restrict__ part) {
  __shared__ float red[8];
  const size_t stride = (size_t)gridDim.x * 256, i0 = (size_t)blockIdx.x * 256 + threadIdx.x;
  float m = 0.f;   // fmaxf drops NaN operands
  for (size_t v = i0; v < n_out / 8; v += stride) {
    const u32x4 x = reinterpret_cast<const u32x4*>(dout)[v];
    const bf16* e = reinterpret_cast<const bf16*>(&x);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f32(e[i])));
  }
  for (size_t v = i0; v < n_fin / 4; v += stride) {
    const f32x4 x = reinterpret_cast<const f32x4*>(dfin)[v];
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(x[i]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane_id() == 0) red[threadIdx.x / 64] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ __launch_bounds__(256) void kda_grad_scale(const float* __restrict__ part, int n, float* __restrict__ gs) {
  __shared__ float red[4];
  float m = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) m = fmaxf(m, part[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane_id() == 0) red[threadIdx.x / 64] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float s = 1.f;
    if (m > 0.f && m <= 3.4e38f) {
      int e;
      (void)frexpf(m, &e);            // m = f 2^e, f in [0.5, 1)
      e = e < -100 ? -100 : (e > 100 ? 100 : e);
      s = ldexpf(1.f, -e);
    }
    gs[0] = s;
    gs[1] = 1.f / s;
  }
}

static hipError_t launch_grad_scale(const Args& a, hipStream_t st) {
  const size_t n_out = (size_t)a.B * a.T * a.H * a.dv;
  const size_t n_fin = a.dfinal ? (size_t)a.N * a.H * a.dk * a.dv : 0;
  KDA_TIMED("kda_grad_absmax", st,
            hipLaunchKernelGGL(kda_grad_absmax, dim3(GS_PARTS), dim3(256), 0, st,
                               reinterpret_cast<const bf16*>(a.dout), n_out, a.dfinal, n_fin, a.gs_part));
  KDA_TIMED("kda_grad_scale", st, hipLaunchKernelGGL(kda_grad_scale, dim3(1), dim3(256), 0, st, a.gs_part, GS_PARTS, a.gscale));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// reverse sequential pass
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV, int DVS>
struct RevLds {
  using OP = typename OpOf<E>::T;
  static constexpr int P = PADE<OP>;
  static constexpr int LDK = DK + P;
  static constexpr int LDT = CH + P;
  static constexpr bool SPLIT = sizeof(OP) == 2;
  // Aqk, Qt and W contract over tokens here, so they are staged transposed (token index
  // contiguous): their MFMA operands are then 16-byte row reads
  static constexpr size_t AQK = 0;                                          // OP    [CH][LDT]  Aqk^T
  static constexpr size_t KHH = AQK + (size_t)CH * LDT * sizeof(OP);        // OP    [CH][LDK]  Kh (hi)
  static constexpr size_t KHL = KHH + (size_t)CH * LDK * sizeof(OP);        // OP    [CH][LDK]  Kh (lo)
  static constexpr size_t QT = KHL + (SPLIT ? (size_t)CH * LDK * sizeof(OP) : 0);  // OP [DK][LDT]  Qt^T
  static constexpr size_t W = QT + (size_t)DK * LDT * sizeof(OP);           // OP    [DK][LDT]  W^T
  static constexpr size_t GAM = W + (size_t)DK * LDT * sizeof(OP);          // float [DK]
  static constexpr size_t DOT = GAM + (size_t)DK * 4;                       // OP    [DVS][LDT]  dO^T slice
  static constexpr size_t DSH = DOT + (size_t)DVS * LDT * sizeof(OP);       // OP    [DVS][LDK]  dS'^T split
  static constexpr size_t DSL = DSH + (size_t)DVS * LDK * sizeof(OP);
  static constexpr size_t DUH = DSL + (size_t)DVS * LDK * sizeof(OP);       // OP    [DVS][LDT]  dU^T split
  static constexpr size_t DUL = DUH + (size_t)DVS * LDT * sizeof(OP);
  static constexpr size_t BYTES = DUL + (size_t)DVS * LDT * sizeof(OP);
  static_assert(BYTES <= 163840, "reverse pass LDS");
};

// Copy of a 64-row tile ([64][COLS], row pitch src_ld) into LDS transposed
// ([COLS][dst_ld]).  Wide tiles of 2-byte elements: a thread loads rows 2p and 2p + 1
// of one 8-column piece and writes the eight (row 2p, row 2p + 1) pairs as 4-byte words;
// the 32 lanes of a half-wave take the 32 row pairs of one piece, so the words they
// write fall in distinct banks.  Otherwise (4-byte elements, or too few pairs to give
// every thread one) a thread loads one row of a piece and the lanes of a wave take 64
// different rows.
template <typename T, int COLS, int NT>
struct TransTile {
  static constexpr bool PAIR = sizeof(T) == 2 && (CH / 2) * (COLS / 8) >= NT;
  static constexpr int EPV = 16 / (int)sizeof(T);            // elements per 16-byte piece
  static constexpr int NP = PAIR ? CH / 2 : CH;              // row units (pairs or rows)
  static constexpr int NI = NP * (COLS / EPV), PER = (NI + NT - 1) / NT;
  u32x4 r0[PER], r1[PAIR ? PER : 1];
  __device__ __forceinline__ void load(const T* __restrict__ src, size_t src_ld) {
    static_for<0, PER>([&](auto I) __attribute__((always_inline)) {
      const int v0 = threadIdx.x + I * NT, v = (NI % NT == 0 || v0 < NI) ? v0 : 0;
      const int p = v % NP, cp = v / NP;
      if constexpr (PAIR) {
        r0[I] = *reinterpret_cast<const u32x4*>(src + (size_t)(2 * p) * src_ld + EPV * cp);
        r1[I] = *reinterpret_cast<const u32x4*>(src + (size_t)(2 * p + 1) * src_ld + EPV * cp);
      } else {
        r0[I] = *reinterpret_cast<const u32x4*>(src + (size_t)p * src_ld + EPV * cp);
      }
    });
  }
  __device__ __forceinline__ void store(T* dst, int dst_ld) const {
    static_for<0, PER>([&](auto I) __attribute__((always_inline)) {
      const int v = threadIdx.x + I * NT;
      if (NI % NT == 0 || v < NI) {
        const int p = v % NP, cp = v / NP;
        if constexpr (PAIR) {
          const unsigned short* a = reinterpret_cast<const unsigned short*>(&r0[I]);
          const unsigned short* b = reinterpret_cast<const unsigned short*>(&r1[I]);
#pragma unroll
          for (int u = 0; u < EPV; ++u)
            *reinterpret_cast<uint32_t*>(dst + (EPV * cp + u) * dst_ld + 2 * p) = (uint32_t)a[u] | ((uint32_t)b[u] << 16);
        } else {
          const T* a = reinterpret_cast<const T*>(&r0[I]);
#pragma unroll
          for (int u = 0; u < EPV; ++u) dst[(EPV * cp + u) * dst_ld + p] = a[u];
        }
      }
    });
  }
};

// LOCAL: a stretch's run from dS' = 0 for the segment scan; only the gradient
// entering the stretch is kept (written where d_init_state goes), no per-chunk
// dS' or dU.
template <typename E, int DK, int DV, int DVS, bool LOCAL = false>
__global__ __launch_bounds__(512) void kda_state_rev(const Args a) {
  using L = RevLds<E, DK, DV, DVS>;
  using OP = typename L::OP;
  using WB = WsBlock<E, DK, DV>;
  constexpr int NT = 512, NSL = DV / DVS;
  constexpr int MTS = DK / 16, NTS = DVS / 16;
  constexpr int NST = MTS * NTS;
  constexpr int SPW = (NST + 7) / 8;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

  int unit, sl;
  if (!xcd_unit(blockIdx.x, NSL, a.N * a.H, unit, sl)) return;
  const int seq = a.seq_order[unit / a.H], h = unit % a.H, H = a.H;   // longest sequences first
  const int n0 = sl * DVS;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), r16 = l & 15, q4 = l >> 4;
  const int c0 = a.seq_chunk0[seq], nch = a.seq_chunk0[seq + 1] - c0;
  int tbeg = 0, tend = 0;
  if (nch > 0) {
    const ChunkInfo first = a.chunks[c0], last = a.chunks[c0 + nch - 1];
    tbeg = first.t0;
    tend = last.t0 + last.len;
  }

  OP* sAqk = reinterpret_cast<OP*>(smem + L::AQK);
  OP* sKhH = reinterpret_cast<OP*>(smem + L::KHH);
  OP* sKhL = reinterpret_cast<OP*>(smem + L::KHL);
  OP* sQt = reinterpret_cast<OP*>(smem + L::QT);
  OP* sW = reinterpret_cast<OP*>(smem + L::W);
  float* sGam = reinterpret_cast<float*>(smem + L::GAM);
  OP* sDOT = reinterpret_cast<OP*>(smem + L::DOT);
  OP* sDSh = reinterpret_cast<OP*>(smem + L::DSH);
  OP* sDSl = reinterpret_cast<OP*>(smem + L::DSL);
  OP* sDUh = reinterpret_cast<OP*>(smem + L::DUH);
  OP* sDUl = reinterpret_cast<OP*>(smem + L::DUL);

  const OP* gAqk = reinterpret_cast<const OP*>(a.wsAqk);
  const char* gKh = reinterpret_cast<const char*>(a.wsKhF);   // per block: hi [CH][DK], then lo (split types)
  const OP* gQt = reinterpret_cast<const OP*>(a.wsQt);
  const OP* gW = reinterpret_cast<const OP*>(a.wsW);
  const float* gGam = a.wsGam;
  const E* gDO = reinterpret_cast<const E*>(a.dout);
  float* gdS = a.wsdS;
  float* gdU = a.wsdU;
  const float* gDFin = a.dfinal;
  float* gDInit = a.dinit;
  const float scale = a.scale;
  const size_t ro = (size_t)H * DV;
  // gradient scale: dO and the caller's dS_final are read times s; d_init_state is
  // stored times 1/s (a stretch's gradient for the segment scan stays scaled)
  const float gs = a.gscale ? a.gscale[0] : 1.f;
  const float gs_fin = a.dfinal_scaled ? 1.f : gs;
  const float gs_inv = (a.gscale && !LOCAL) ? a.gscale[1] : 1.f;

  // every load is issued before the first use (a use between them would wait for each in turn)
  f32x4 dS[SPW];
  const size_t st_off = ((size_t)seq * H + h) * DK * DV;
  if (gDFin) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = min(w + 8 * i, NST - 1), mt = t % MTS, nt = t / MTS;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) dS[i][ii] = gDFin[st_off + (size_t)(16 * mt + 4 * q4 + ii) * DV + n0 + 16 * nt + r16];
    }
#pragma unroll
    for (int i = 0; i < SPW; ++i) dS[i] = w + 8 * i < NST ? dS[i] * gs_fin : zero4();
  } else {
#pragma unroll
    for (int i = 0; i < SPW; ++i) dS[i] = zero4();
  }

  // dO slice: 64 token rows x DVS columns of the input, rows past the chunk zeroed
  constexpr int EPV = 16 / (int)sizeof(E), VPR = DVS / EPV, NVO = CH * VPR;
  struct Stage {
    TransTile<OP, CH, NT> aqk;
    TileCopy<OP, CH, DK, NT> khh;
    TileCopy<OP, (L::SPLIT ? CH : 1), (L::SPLIT ? DK : 16 / sizeof(OP)), NT> khl;
    TransTile<OP, DK, NT> qt;
    TransTile<OP, DK, NT> w;
    TileCopy<float, 1, DK, NT> gam;
    u32x4 dov;  // one 16-byte piece of the dO slice (threads < NVO)
    int dolen;
  };
  static_assert(NVO <= NT, "dO slice staging");
  Stage st0, st1;
  auto blk_of = [&](int n) { return (size_t)(c0 + n) * H + h; };
  // a chunk's operands -> registers, in two parts issued at different points of a step
  // (the memory queue then never holds all of them ahead of the step's stores)
  auto stage_load_a = [&](Stage& p, int n) __attribute__((always_inline)) {
    const size_t b = blk_of(n);
    p.aqk.load(gAqk + b * WB::AQK, CH);
    const OP* kb = reinterpret_cast<const OP*>(gKh + b * WB::KHF * sizeof(float));
    p.khh.load(kb, DK);
    if constexpr (L::SPLIT) p.khl.load(kb + CH * DK, DK);
  };
  auto stage_load = [&](Stage& p, int n) __attribute__((always_inline)) {
    const size_t b = blk_of(n);
    p.qt.load(gQt + b * WB::QT, DK);
    p.w.load(gW + b * WB::W, DK);
    p.gam.load(gGam + b * WB::GAM, DK);
    const int t0 = tbeg + n * CH;
    p.dolen = min(CH, tend - t0);
    const int v = tid < NVO ? tid : 0;
    const int row = v / VPR, cv = v % VPR;
    const int rr = row < p.dolen ? row : 0;  // rows past the chunk re-read row 0 (zeroed on store)
    p.dov = *reinterpret_cast<const u32x4*>(gDO + (size_t)(t0 + rr) * ro + (size_t)h * DV + n0 + cv * EPV);
  };
  auto stage_store = [&](const Stage& p) __attribute__((always_inline)) {
    p.aqk.store(sAqk, L::LDT);
    p.khh.store(sKhH, L::LDK);
    if constexpr (L::SPLIT) p.khl.store(sKhL, L::LDK);
    p.qt.store(sQt, L::LDT);
    p.w.store(sW, L::LDT);
    p.gam.store(sGam, DK);
    if (tid < NVO) {
      const int row = tid / VPR, cv = tid % VPR;
      const bool ok = row < p.dolen;
      const E* e = reinterpret_cast<const E*>(&p.dov);
#pragma unroll
      for (int i = 0; i < EPV; ++i) sDOT[(cv * EPV + i) * L::LDT + row] = cvt<OP>(ok ? gs * f32(e[i]) : 0.f);
    }
  };

  auto chunk = [&](int n, Stage& ld, const Stage& nx) __attribute__((always_inline)) {
    // dS' (gradient of the state leaving chunk n) -> LDS split, and -> workspace fp32
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = w + 8 * i, mt = t % MTS, nt = t / MTS;
      if (t < NST) {
        const int off = (16 * nt + r16) * L::LDK + 16 * mt + 4 * q4;
        store4_split<OP>(sDSh + off, sDSl + off, dS[i][0], dS[i][1], dS[i][2], dS[i][3]);
        if constexpr (!LOCAL) {
          float* dst = gdS + blk_of(n) * WB::DS + (size_t)(16 * mt + 4 * q4) * DV + n0 + 16 * nt + r16;  // [DK][DV]
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) dst[(size_t)ii * DV] = dS[i][ii];
        }
      }
    }
    __syncthreads();
    // chunk n - 2 -> registers, first part, issued after this step's dS' stores: stores
    // issued behind the loads would wait for them in the memory queue
    stage_load_a(ld, max(n - 2, 0));

    // dU = scale Aqk^T dO + Kh dS' : tiles (token tile tt, value tile nt) dealt to all eight waves
    constexpr int NDU = 4 * NTS, DPW = (NDU + 7) / 8;
#pragma unroll
    for (int j = 0; j < DPW; ++j) {
      const int u = w + 8 * j, tt = u % 4, nt = u / 4;
      if (u < NDU) {
        f32x4 x1 = zero4(), x2 = zero4();
#pragma unroll
        for (int k = 0; k < CH; k += 32)
          x1 = mma(frag_row<OP>(sAqk, L::LDT, 16 * tt + r16, k + 8 * q4),
                   frag_row<OP>(sDOT, L::LDT, 16 * nt + r16, k + 8 * q4), x1);
#pragma unroll
        for (int k = 0; k < DK; k += 32)
          x2 = mma_ss(sfrag_pair<OP>(sKhH, sKhL, L::LDK, 16 * tt + r16, k + 8 * q4),
                      sfrag_pair<OP>(sDSh, sDSl, L::LDK, 16 * nt + r16, k + 8 * q4), x2);
        const f32x4 du = scale * x1 + x2;
        const int off = (16 * nt + r16) * L::LDT + 16 * tt + 4 * q4;
        store4_split<OP>(sDUh + off, sDUl + off, du[0], du[1], du[2], du[3]);
        if constexpr (!LOCAL) {
          float* dst = gdU + blk_of(n) * WB::DU + (size_t)(16 * tt + 4 * q4) * DV + n0 + 16 * nt + r16;  // [CH][DV]
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) dst[(size_t)ii * DV] = du[ii];
        }
      }
    }
    // scale Qt^T dO for this wave's state tiles (independent of dU)
    f32x4 qd[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = w + 8 * i, mt = t % MTS, nt = t / MTS;
      qd[i] = zero4();
      if (t < NST) {
#pragma unroll
        for (int k = 0; k < CH; k += 32)
          qd[i] = mma(frag_row<OP>(sQt, L::LDT, 16 * mt + r16, k + 8 * q4),
                      frag_row<OP>(sDOT, L::LDT, 16 * nt + r16, k + 8 * q4), qd[i]);
      }
    }
    __syncthreads();
    stage_load(ld, max(n - 2, 0));   // second part, after this step's dU stores
    // dS = Gamma_C dS' + scale Qt^T dO - W^T dU
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = w + 8 * i, mt = t % MTS, nt = t / MTS;
      if (t < NST) {
        f32x4 x = zero4();
#pragma unroll
        for (int k = 0; k < CH; k += 32)
          x = mma_ps(frag_row<OP>(sW, L::LDT, 16 * mt + r16, k + 8 * q4),
                     sfrag_pair<OP>(sDUh, sDUl, L::LDT, 16 * nt + r16, k + 8 * q4), x);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          dS[i][ii] = sGam[16 * mt + 4 * q4 + ii] * dS[i][ii] + scale * qd[i][ii] - x[ii];
      }
    }
    __syncthreads();
    if (n > 0) stage_store(nx);
  };

  if (nch > 0) {
    stage_load_a(st0, nch - 1);
    stage_load(st0, nch - 1);
    stage_store(st0);
    stage_load_a(st1, max(nch - 2, 0));
    stage_load(st1, max(nch - 2, 0));
  }
  // chunks in reverse order; stage sets alternate so their registers stay static
  int n = nch - 1;
  for (; n >= 1; n -= 2) {
    chunk(n, st0, st1);
    chunk(n - 1, st1, st0);
  }
  if (n == 0) chunk(0, st0, st1);

  if (gDInit) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = w + 8 * i, mt = t % MTS, nt = t / MTS;
      if (t < NST) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int ch = 16 * mt + 4 * q4 + ii, col = n0 + 16 * nt + r16;
          gDInit[st_off + (size_t)ch * DV + col] = gs_inv * dS[i][ii];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// chunk-parallel gradients: one workgroup per chunk-head, 8 waves
// ---------------------------------------------------------------------------
// Wave w owns token tile tw = w & 3 (rows 16tw..16tw+15) and half hf = w >> 2
// of the column tiles of every product it computes; over the key channels, that
// half is the tiles 2 jj + hf (the even or the odd ones), so the two halves of
// every pass jj cover 32 adjacent channels and a token row's gradient stores for
// them land in one 64-byte segment.
//
// Phase A walks the value dimension in quarters of 32 columns and accumulates
// the contractions over it (dAqk = scale tril(dO U^T), dT_U = dU V^T,
// dQS = dO S^T, dKh = U dS'^T, dW = -dU S^T), writes dV = beta T^T dU, and
// the value sums of V * T^T dU (for dbeta) and dS' * S (dGamma_C).  Two
// quarters are in flight: the one after next is loaded into registers while the
// current one is multiplied.
//
// Phase B works over tokens and channels: T^T dW, dT, dA = -strict(T^T dT T^T),
// the gated products with per-block reference rows, and the assembly of dq,
// dk, dg, dbeta; dlog_alpha is the reverse cumulative sum of dg over the chunk.
// dQS, dKh and dT_U stay in the accumulator registers of phase A, in the same
// tile layout phase B consumes them in.
template <typename E, int DK, int DV>
struct BwdLds {
  using OP = typename OpOf<E>::T;
  static constexpr int PE = PADE<E>, PO = PADE<OP>;
  static constexpr int QC = 32;                      // value columns per quarter
  static constexpr bool SPLIT = sizeof(OP) == 2;     // lo halves exist only for 2-byte operands
  static constexpr size_t OPB = sizeof(OP);
  // phase A: quarters with the value column contiguous, so every MFMA operand
  // (contraction over the value dimension) is one 16-byte row read
  static constexpr int LSV = QC + PO;   // OP [DK][LSV] S, dS';  [CH][LSV] U, dU, dO, V
  static constexpr size_t A_SH = 0;                                  // S in the operand type
  static constexpr size_t A_DSH = A_SH + (size_t)DK * LSV * OPB;      // dS' split (hi, lo)
  static constexpr size_t A_DSL = A_DSH + (size_t)DK * LSV * OPB;
  static constexpr size_t A_UH = A_DSL + (SPLIT ? (size_t)DK * LSV * OPB : 0);
  static constexpr size_t A_UL = A_UH + (size_t)CH * LSV * OPB;
  static constexpr size_t A_DUH = A_UL + (SPLIT ? (size_t)CH * LSV * OPB : 0);
  static constexpr size_t A_DUL = A_DUH + (size_t)CH * LSV * OPB;
  static constexpr size_t A_DO = A_DUL + (SPLIT ? (size_t)CH * LSV * OPB : 0);
  static constexpr size_t A_V = A_DO + (size_t)CH * LSV * OPB;
  static constexpr size_t A_END = A_V + (size_t)CH * LSV * OPB;
  // phase B (shares the first region with phase A)
  static constexpr int LDG = DK + 4;    // float [CH][LDG]  g, later dg
  static constexpr int LDK = DK + PE;   // E     [CH][LDK]  k, q
  static constexpr int LDO = DK + PO;   // OP    [CH][LDO]  dW, K+
  static constexpr int LDT = CH + PO;   // OP    [CH][LDT]  T, Y
  static constexpr int LDA = CH + 4;    // float [CH][LDA]  dT
  using SE = typename std::conditional<sizeof(E) == 4, float, bf16>::type;   // gated-product operands
  static constexpr bool SSPLIT = sizeof(SE) == 2;
  static constexpr int LDQ = CH + PADE<SE>;   // SE [..][LDQ]  split dAqk / dG rows, decayed q/k tables
  static constexpr int LDR = CH + 4;          // float [..][LDR]  decayed k table
  static constexpr size_t G = 0;
  static constexpr size_t K = G + (size_t)CH * LDG * 4;
  static constexpr size_t Q = K + (size_t)CH * LDK * sizeof(E);
  static constexpr size_t B_END = Q + (size_t)CH * LDK * sizeof(E);
  static constexpr size_t UNION = A_END > B_END ? A_END : B_END;
  // both phases
  static constexpr size_t T = UNION;                                  // OP    [CH][LDT]  T^T
  static constexpr size_t QSZ = (size_t)CH * LDQ * sizeof(SE);       // one SE [CH][LDQ] array
  static constexpr size_t A1 = T + (size_t)CH * LDT * OPB;            // SE hi, lo [CH][LDQ]  scale tril(dO U^T)
  static constexpr size_t A2 = A1 + (SSPLIT ? 2 : 1) * QSZ;           // float [CH][LDA] dT, then SE hi, lo dG
  static constexpr size_t A2SZ = (size_t)CH * LDA * 4 > (SSPLIT ? 2 : 1) * QSZ ? (size_t)CH * LDA * 4
                                                                              : (SSPLIT ? 2 : 1) * QSZ;
  static constexpr size_t DW = A2 + A2SZ;                             // OP    [CH][LDO]  dW (Y after it is dead)
  static constexpr size_t KP = DW + (size_t)CH * LDO * OPB;           // OP    [CH][LDO]  K+
  static constexpr size_t BETA = KP + (size_t)CH * LDO * OPB;         // float [CH]
  static constexpr size_t RED = BETA + CH * 4;                        // float [512]  scan / column-sum partials
  static constexpr size_t DGAM = RED + 512 * (sizeof(E) == 4 ? 8 : 4);   // float [DK]  dGamma_C (fp32 inputs:
                                                                          // RED holds the scan's fp64 part sums)
  static constexpr size_t BV = DGAM + DK * 4;                         // float [2][CH] rowsum(V * T^T dU) halves
  static constexpr size_t DBP = BV + 2 * CH * 4;                      // float [2][CH] dbeta halves
  static constexpr size_t NRM = DBP + 2 * CH * 4;                     // float [2][CH] 1/|q_r|, 1/|k_r| (qk_norm)
  static constexpr size_t NDOT = NRM + 2 * CH * 4;                    // float [2][2][CH] q^.dq^, k^.dk^ halves
  static constexpr size_t END0 = NDOT + 4 * CH * 4;
  static constexpr size_t Y = DW;                                     // OP hi, lo [CH][LDT] Y^T (dW, K+ dead by then)
  static constexpr size_t YL = Y + (size_t)CH * LDT * OPB;
  static_assert(2 * (size_t)CH * LDT <= 2 * (size_t)CH * LDO, "split Y fits in the dW and K+ regions");
  // gated products, per pass of 32 channels: fp32 tables [channel][token] of
  // q_r e^{g_r - g_m(R)}, k_r e^{g_r - g_m(R)} (row side) and k_i e^{g_m(C) - g_i}
  // (column side), R, C the tokens' 8-token groups.  They reuse the dW and K+ regions
  // (dead by then) where those are large enough (dk = 128), else they follow the rest.
  static constexpr int TC = 32;
  static constexpr size_t TAB1 = (size_t)TC * LDR * 4;
  static constexpr size_t TAB_SZ = 3 * TAB1;
  static constexpr bool TAB_REUSE = TAB_SZ <= 2 * (size_t)CH * LDO * OPB;
  static constexpr size_t TQ = TAB_REUSE ? DW : END0;
  static constexpr size_t TK = TQ + TAB1;
  static constexpr size_t KR = TK + TAB1;
  static constexpr size_t BYTES1 = TAB_REUSE ? END0 : END0 + TAB_SZ;
  // a second table set, so the next pass's tables are built while the current pass reads
  // its own: T^T's block (dead after dA) holds one table; the rest go into the dW and K+
  // regions past the first set (or into them, when the first set follows the rest), and
  // what is left past the end of the layout
  static constexpr size_t DWKP = 2 * (size_t)CH * LDO * OPB;   // dW and K+ regions together
  static constexpr size_t TQ2 = T;
  static constexpr size_t TK2 = TAB_REUSE ? DW + TAB_SZ : DW;
  static constexpr size_t KR2 = TAB_REUSE ? (DW + TAB_SZ + TAB1 <= DW + DWKP ? BYTES1 : 0) : DW + TAB1;
  static constexpr size_t BYTES2 = TAB_REUSE ? BYTES1 + TAB1 : BYTES1;
  static constexpr bool TDB = (size_t)CH * LDT * OPB >= TAB1 && BYTES2 <= 163840 &&
                              (TAB_REUSE ? DW + TAB_SZ + TAB1 <= DW + DWKP : 2 * TAB1 <= DWKP);
  static constexpr size_t BYTES = TDB ? BYTES2 : BYTES1;
  static_assert(KR % 16 == 0 && TK % 16 == 0 && TQ % 16 == 0, "table rows stay 16-byte aligned");
  static_assert(KR2 % 16 == 0 && TK2 % 16 == 0 && TQ2 % 16 == 0, "table rows stay 16-byte aligned");
  static_assert(BYTES <= 163840, "backward chunk kernel LDS");
  static_assert(RED % 8 == 0, "fp64 scan partials stay 8-byte aligned");
  static_assert(A_END % 16 == 0 && B_END % 16 == 0, "LDS regions stay 16-byte aligned");
};

// QKN: q and k rows are L2-normalised on load and dq, dk go through the norm's
// chain rule at the end (KDA_FLAG_QK_L2NORM).  PATH 0 takes the chunk-heads the prep
// left unflagged in a.steep, PATH 1 the flagged ones (decayed products through
// 8-token groups); two instantiations keep the usual path's registers free of the
// other one's.
template <typename E, typename O, int DK, int DV, bool QKN, int PATH>
__global__ __launch_bounds__(512) void kda_bwd_chunk(const Args a) {
  using L = BwdLds<E, DK, DV>;
  using OP = typename L::OP;
  using WB = WsBlock<E, DK, DV>;
  constexpr int NT = 512, NKT = DK / 16, NKH = NKT / 2, QC = L::QC, NQ = DV / QC;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  const int j = blockIdx.x, h = blockIdx.y, H = a.H;
  const ChunkInfo ci = a.chunks[j];
  if (ci.len <= 0) return;
  if ((a.steep[(size_t)j * H + h] != 0) != (PATH == 1)) return;
  const int len = ci.len;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), r16 = l & 15, q4 = l >> 4;
  // token tile tw and column half hf of this wave.  Waves w and w + 4 share a
  // SIMD; the second half takes the tiles in reverse order, so each SIMD pairs a
  // tile near the top of the chunk with one near the bottom and the triangular
  // products load the four SIMDs evenly.
  const int hf = w >> 2, tw = hf ? 3 - (w & 3) : (w & 3), kq = 8 * q4;
  const size_t blk = (size_t)j * H + h;
  const size_t rk = (size_t)H * DK, rv = (size_t)H * DV;
  const float scale = a.scale;

  OP* sSh = reinterpret_cast<OP*>(smem + L::A_SH);
  OP* sDSh = reinterpret_cast<OP*>(smem + L::A_DSH);
  OP* sDSl = reinterpret_cast<OP*>(smem + L::A_DSL);
  OP* sUh = reinterpret_cast<OP*>(smem + L::A_UH);
  OP* sUl = reinterpret_cast<OP*>(smem + L::A_UL);
  OP* sDUh = reinterpret_cast<OP*>(smem + L::A_DUH);
  OP* sDUl = reinterpret_cast<OP*>(smem + L::A_DUL);
  OP* sDO = reinterpret_cast<OP*>(smem + L::A_DO);
  OP* sV = reinterpret_cast<OP*>(smem + L::A_V);
  float* sG = reinterpret_cast<float*>(smem + L::G);
  E* sK = reinterpret_cast<E*>(smem + L::K);
  E* sQ = reinterpret_cast<E*>(smem + L::Q);
  OP* sTT = reinterpret_cast<OP*>(smem + L::T);   // T^T: sTT[i][r] = T[r][i]
  using SE = typename L::SE;   // gated-product operands: split bf16 (fp32 on the fp32 path)
  SE* sA1h = reinterpret_cast<SE*>(smem + L::A1);   // scale tril(dO U^T), split
  SE* sA1l = sA1h + CH * L::LDQ;
  float* sA2 = reinterpret_cast<float*>(smem + L::A2);   // dT
  SE* sA2h = reinterpret_cast<SE*>(smem + L::A2);   // dG, split (after dT is dead)
  SE* sA2l = sA2h + CH * L::LDQ;
  float* tQ = reinterpret_cast<float*>(smem + L::TQ);
  float* tK = reinterpret_cast<float*>(smem + L::TK);
  float* tKR = reinterpret_cast<float*>(smem + L::KR);
  float* tQ2 = reinterpret_cast<float*>(smem + L::TQ2);   // second set (used when L::TDB)
  float* tK2 = reinterpret_cast<float*>(smem + L::TK2);
  float* tKR2 = reinterpret_cast<float*>(smem + L::KR2);
  // x as a split pair hi + lo (hi only on the fp32 path)
  auto put_split = [&](SE* hi, SE* lo, int idx, float x) __attribute__((always_inline)) {
    if constexpr (L::SSPLIT) {
      const SE hv = (SE)x;
      hi[idx] = hv;
      lo[idx] = (SE)(x - (float)hv);
    } else {
      hi[idx] = x;
    }
  };
  OP* sDW = reinterpret_cast<OP*>(smem + L::DW);
  OP* sY = reinterpret_cast<OP*>(smem + L::Y);
  OP* sYl = reinterpret_cast<OP*>(smem + L::YL);
  OP* sKp = reinterpret_cast<OP*>(smem + L::KP);
  float* sBeta = reinterpret_cast<float*>(smem + L::BETA);
  float* sRed = reinterpret_cast<float*>(smem + L::RED);
  float* sDGam = reinterpret_cast<float*>(smem + L::DGAM);
  float* sBv = reinterpret_cast<float*>(smem + L::BV);
  float* sDbp = reinterpret_cast<float*>(smem + L::DBP);
  float* sNrm = reinterpret_cast<float*>(smem + L::NRM);
  float* sDot = reinterpret_cast<float*>(smem + L::NDOT);
  constexpr bool qk_norm = QKN;
  // normalised q and k values: raw row element times the row's 1/|x| (1 without QKN)
  auto qn = [&](int r, int c) __attribute__((always_inline)) {
    if constexpr (QKN) return f32(sQ[r * L::LDK + c]) * sNrm[r];
    else return f32(sQ[r * L::LDK + c]);
  };
  auto kn = [&](int r, int c) __attribute__((always_inline)) {
    if constexpr (QKN) return f32(sK[r * L::LDK + c]) * sNrm[CH + r];
    else return f32(sK[r * L::LDK + c]);
  };

  const E* qh = reinterpret_cast<const E*>(a.q) + (size_t)ci.t0 * rk + (size_t)h * DK;
  const E* kh = reinterpret_cast<const E*>(a.k) + (size_t)ci.t0 * rk + (size_t)h * DK;
  const E* lh = reinterpret_cast<const E*>(a.la) + (size_t)ci.t0 * rk + (size_t)h * DK;
  const E* vh = reinterpret_cast<const E*>(a.v) + (size_t)ci.t0 * rv + (size_t)h * DV;
  const E* doh = reinterpret_cast<const E*>(a.dout) + (size_t)ci.t0 * rv + (size_t)h * DV;
  const E* bh = reinterpret_cast<const E*>(a.beta) + (size_t)ci.t0 * H + h;
  const float* gS = a.wsS + blk * WB::S;
  const float* gdS = a.wsdS + blk * WB::DS;
  const float* gU = a.wsU + blk * WB::U;
  const float* gdU = a.wsdU + blk * WB::DU;
  const OP* gT = reinterpret_cast<const OP*>(a.wsT) + blk * WB::TT;
  const float* gGm = a.wsG + blk * WB::G;
  O* gdV = reinterpret_cast<O*>(a.dv_) + (size_t)ci.t0 * rv + (size_t)h * DV;
  // gradient scale: dO is read times s, every gradient stored times 1/s
  const float gs = a.gscale ? a.gscale[0] : 1.f;
  const float gs_inv = a.gscale ? a.gscale[1] : 1.f;

  // phase B's inputs (q, k, log_alpha rows), loaded during the last value quarter
  TileCopy<E, CH, DK, NT> pk, pq, pl;
  // Gamma_C of the channel whose dg_C this thread finishes in the tail (read now:
  // a load issued after the gradient stores would wait for them to drain), and beta
  // of row tid.  Both are issued ahead of the tile loads, without a branch, and not
  // touched until used, so no wait for them holds up the loads behind them.
  const float gam_c = a.wsGam[blk * WB::GAM + min(max(tid - 64, 0), DK - 1)];   // used by threads 64 .. 64 + DK - 1
  const E beta_raw = bh[(size_t)min(tid % CH, len - 1) * H];                    // rows past the chunk: zeroed when staged
  __builtin_amdgcn_sched_barrier(0);   // keep the two loads ahead of the tile loads

  // ---- phase A staging: contractions over the value dimension, a quarter of the columns at a time
  struct QStage {
    TileCopy<float, DK, QC, NT> s, ds;   // the same shape and type: a thread holds the same elements of both
    TileCopy<float, CH, QC, NT> u, du;
    TileCopy<E, CH, QC, NT> dov, vv;
  };
  // two quarters in flight: quarter qq sits in stage qq % 2
  QStage qst[2];
  auto qload = [&](QStage& qs, int qq) __attribute__((always_inline)) {
    const int cq = qq * QC;
    qs.s.load(gS + cq, DV);
    qs.ds.load(gdS + cq, DV);
    qs.u.load(gU + cq, DV);
    qs.du.load(gdU + cq, DV);
    qs.dov.load(doh + cq, rv, len);   // rows past the chunk are not read; they are zeroed on store
    qs.vv.load(vh + cq, rv, len);
  };

  // ---- T^T -> LDS (operand type), beta; the first quarter's loads are in flight meanwhile
  {
    TileCopy<OP, CH, CH, NT> tt;
    tt.load(gT, CH);
    qload(qst[0], 0);
    if (NQ > 1) qload(qst[1], 1);
    constexpr int EPV = 16 / (int)sizeof(OP);
    static_for<0, decltype(tt)::PER>([&](auto I) __attribute__((always_inline)) {
      const int v = tid + I * NT;
      if (decltype(tt)::NV % NT == 0 || v < decltype(tt)::NV) {
        const int row = v / (CH / EPV), c0 = (v % (CH / EPV)) * EPV;
        const OP* x = reinterpret_cast<const OP*>(&tt.r[I]);
#pragma unroll
        for (int u = 0; u < EPV; ++u) sTT[(c0 + u) * L::LDT + row] = x[u];
      }
    });
  }
  if (tid < CH) sBeta[tid] = tid < len ? f32(beta_raw) : 0.f;

  // ---- phase A
  f32x4 accA[2], accT[2], accQ[NKH], accK[NKH], accW[NKH];
#pragma unroll
  for (int i = 0; i < 2; ++i) accA[i] = accT[i] = zero4();
#pragma unroll
  for (int i = 0; i < NKH; ++i) accQ[i] = accK[i] = accW[i] = zero4();
  float bv[4] = {0.f, 0.f, 0.f, 0.f};
  constexpr int GPER = TileCopy<float, DK, QC, NT>::PER;
  float gp[GPER];   // partial dGamma_C of the rows this thread holds in the quarter tiles
#pragma unroll
  for (int i = 0; i < GPER; ++i) gp[i] = 0.f;

#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) {
    const int cq = qq * QC;
    QStage& qs = qst[qq & 1];
    __syncthreads();  // the previous quarter's LDS reads are done
    qs.s.template store_cvt<OP>(sSh, L::LSV, DK);
    qs.ds.template store_split<OP>(sDSh, sDSl, L::LSV);
    qs.u.template store_split<OP>(sUh, sUl, L::LSV);
    qs.du.template store_split<OP>(sDUh, sDUl, L::LSV);
    qs.dov.template store_map<OP>(sDO, L::LSV, len, [gs](float x) { return gs * x; });
    qs.vv.template store_cvt<OP>(sV, L::LSV, len);
    // dGamma_C = value sums of dS' * S, in fp32 from the registers the quarter was loaded
    // into (before the next quarter's loads reuse them): a thread holds the same 4-column pieces of S and dS'
    static_for<0, decltype(qs.s)::PER>([&](auto I) __attribute__((always_inline)) {
      const float* x = reinterpret_cast<const float*>(&qs.s.r[I]);
      const float* y = reinterpret_cast<const float*>(&qs.ds.r[I]);
      gp[I] += (x[0] * y[0] + x[1] * y[1]) + (x[2] * y[2] + x[3] * y[3]);
    });
    __syncthreads();
    // the quarter after next, and in the last quarter phase B's inputs, issued once the
    // barrier has passed (issued before it, they hold up the waves still storing)
    if (qq + 2 < NQ) qload(qs, qq + 2);
    if (qq + 1 == NQ) {
      pk.load(kh, rk, len);
      pq.load(qh, rk, len);
      pl.load(lh, rk, len);
    }
    const Frag<OP> fdo = frag_row<OP>(sDO, L::LSV, 16 * tw + r16, kq);
    const SFrag<OP> fdu = sfrag_pair<OP>(sDUh, sDUl, L::LSV, 16 * tw + r16, kq);
    const SFrag<OP> fu = sfrag_pair<OP>(sUh, sUl, L::LSV, 16 * tw + r16, kq);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int nt = 2 * hf + jj;
      accA[jj] = mma_ps(fdo, sfrag_pair<OP>(sUh, sUl, L::LSV, 16 * nt + r16, kq), accA[jj]);
      accT[jj] = mma_sp(fdu, frag_row<OP>(sV, L::LSV, 16 * nt + r16, kq), accT[jj]);
    }
#pragma unroll
    for (int jj = 0; jj < NKH; ++jj) {
      const int nt = 2 * jj + hf;
      // S in the operand type: these products tolerate its rounding (dGamma_C, which
      // does not, comes from the fp32 registers above)
      const Frag<OP> fs = frag_row<OP>(sSh, L::LSV, 16 * nt + r16, kq);
      accQ[jj] = mma(fdo, fs, accQ[jj]);
      accW[jj] = mma_sp(fdu, fs, accW[jj]);
      accK[jj] = mma_ss(fu, sfrag_pair<OP>(sDSh, sDSl, L::LSV, 16 * nt + r16, kq), accK[jj]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // dV = beta T^T dU for token tile tw and the quarter's column tile hf
    {
      f32x4 x = zero4();
#pragma unroll
      for (int k = 0; k < CH; k += 32)
        x = mma_ps(frag_row<OP>(sTT, L::LDT, 16 * tw + r16, k + kq),
                   sfrag_col_pair<OP>(sDUh, sDUl, L::LSV, 16 * hf + r16, k + kq), x);
      f32x4 y;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 16 * tw + 4 * q4 + ii, col = 16 * hf + r16;
        bv[ii] += f32(sV[r * L::LSV + col]) * x[ii];   // reduced over the column lanes after phase A
        y[ii] = gs_inv * (sBeta[r] * x[ii]);
      }
      // dV after a quad transpose: row 16 tw + 4 q4 + (r16 & 3), 4 columns
      y = quad_transpose(y);
      const int rt = 16 * tw + 4 * q4 + (r16 & 3);
      if (rt < len) store4<O>(gdV + (size_t)rt * rv + cq + 16 * hf + (r16 & ~3), y[0], y[1], y[2], y[3]);
    }
  }
  __syncthreads();  // phase A's LDS reads are done; its region is reused below

  // ---- hand-over: dAqk, dW to LDS; partial sums; phase B inputs to LDS
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int rr = 16 * tw + 4 * q4 + ii;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int cc = 16 * (2 * hf + jj) + r16;
      put_split(sA1h, sA1l, rr * L::LDQ + cc, cc <= rr ? scale * accA[jj][ii] : 0.f);
    }
#pragma unroll
    for (int jj = 0; jj < NKH; ++jj) sDW[rr * L::LDO + 16 * (2 * jj + hf) + r16] = cvt<OP>(-accW[jj][ii]);
    const float p = lane_sum16(bv[ii]);
    if (r16 == 0) sBv[hf * CH + rr] = p;
  }
  {
    // a row's QC / 4 column pieces sit in consecutive lanes
    constexpr int VPR = QC / 4;
    static_for<0, GPER>([&](auto I) __attribute__((always_inline)) {
      static_assert(VPR == 8, "a row's pieces fill one half-row of lanes");
      const float p = lane_sum8(gp[I]);
      const int v = tid + I * NT;
      if (v % VPR == 0 && v < DK * VPR) sDGam[v / VPR] = p;
    });
  }
  float gGram[2][4];   // this wave's tiles of the un-beta strict Gram (for dbeta)
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) gGram[jj][ii] = gGm[(16 * tw + 4 * q4 + ii) * CH + 16 * (2 * hf + jj) + r16];
  if constexpr (qk_norm) {   // each row's 1/|x|; the raw rows stay in LDS and every use scales them
    float scq[decltype(pq)::PER], sck[decltype(pk)::PER];
    pq.row_inv_norms(L2N_EPS, scq);
    pk.row_inv_norms(L2N_EPS, sck);
#pragma unroll
    for (int I = 0; I < decltype(pq)::PER; ++I) {
      int row;
      if (pq.row_leader(I, row)) {
        sNrm[row] = scq[I];
        sNrm[CH + row] = sck[I];
      }
    }
  }
  pk.template store_cvt<E>(sK, L::LDK, len);
  pq.template store_cvt<E>(sQ, L::LDK, len);
  if (a.gate_ls)   // raw gate x -> log alpha = logsigmoid(x)
    pl.template store_map<float>(sG, L::LDG, len, [](float x) { return floor_log_alpha(logsigmoid(x)); });
  else
    pl.template store_map<float>(sG, L::LDG, len, [](float x) { return floor_log_alpha(x); });
  __syncthreads();
  // cumulative sum of log_alpha over the chunk (per channel, NT / DK row parts); for
  // fp32 inputs in fp64 with one rounding of each g to fp32, as in the forward's prep
  constexpr int NSPLIT = NT / DK, RPS = CH / NSPLIT;
  // each thread finishes the rows of its part and forms K+ = k e^g for them at once
  auto put_kp = [&](int rr, int c, float g) __attribute__((always_inline)) {
    sKp[rr * L::LDO + c] = cvt<OP>(kn(rr, c) * __expf(g));
  };
  if constexpr (sizeof(E) == 4) {
    double* sTot = reinterpret_cast<double*>(sRed);
    const int c = tid % DK, s = tid / DK;
    double tot = 0.0;
#pragma unroll
    for (int rr = s * RPS; rr < (s + 1) * RPS; ++rr) tot += (double)sG[rr * L::LDG + c];
    sTot[s * DK + c] = tot;
    __syncthreads();
    double acc = 0.0;
    for (int s2 = 0; s2 < s; ++s2) acc += sTot[s2 * DK + c];
#pragma unroll
    for (int rr = s * RPS; rr < (s + 1) * RPS; ++rr) {
      acc += (double)sG[rr * L::LDG + c];
      const float g = (float)acc;
      sG[rr * L::LDG + c] = g;
      put_kp(rr, c, g);
    }
  } else {
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
      for (int rr = s * RPS; rr < (s + 1) * RPS; ++rr) {
        const float g = sG[rr * L::LDG + c] + off;
        sG[rr * L::LDG + c] = g;
        put_kp(rr, c, g);
      }
    }
  }
  __syncthreads();

  // per-lane C-tile layout below: rows 16tw + 4q4 + ii, columns 16nt + r16
  // ---- T^T dW (channel tiles 2 jj + hf) and rowsum(K+ * T^T dW)
  f32x4 tdw[NKH];
  float dbeta[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jj = 0; jj < NKH; ++jj) {
    const int nt = 2 * jj + hf;
    f32x4 x = zero4();
#pragma unroll
    for (int k = 0; k < CH; k += 32)
      x = mma(frag_row<OP>(sTT, L::LDT, 16 * tw + r16, k + kq), frag_col<OP>(sDW, L::LDO, 16 * nt + r16, k + kq), x);
    tdw[jj] = x;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int rr = 16 * tw + 4 * q4 + ii, cc = 16 * nt + r16;
      dbeta[ii] += kn(rr, cc) * __expf(sG[rr * L::LDG + cc]) * x[ii];
    }
  }
  // ---- dT = (dW K+^T + dU V^T) diag(beta), column tiles 2hf, 2hf+1 -> sA2
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int nt = 2 * hf + jj;
    f32x4 x = zero4();
#pragma unroll
    for (int k = 0; k < DK; k += 32)
      x = mma(frag_row<OP>(sDW, L::LDO, 16 * tw + r16, k + kq), frag_row<OP>(sKp, L::LDO, 16 * nt + r16, k + kq), x);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int rr = 16 * tw + 4 * q4 + ii, cc = 16 * nt + r16;
      sA2[rr * L::LDA + cc] = (x[ii] + accT[jj][ii]) * sBeta[cc];
    }
  }
  __syncthreads();  // dT complete; dW and K+ are dead
  // ---- Y = dT T^T -> sY.  dT and Y are split operands: dA reaches dg through both
  // sides of every gated product, and dlog alpha sums their nearly cancelling difference
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int nt = 2 * hf + jj;
    f32x4 x = zero4();
#pragma unroll
    for (int k = 0; k < CH; k += 32) {
      float y8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) y8[u] = sA2[(16 * tw + r16) * L::LDA + k + kq + u];
      x = mma_sp(sfrag_from<OP>(y8), frag_col<OP>(sTT, L::LDT, 16 * nt + r16, k + kq), x);
    }
    // stored transposed (Y^T[col][row]): this lane's four rows are one 8-byte run, and dA
    // below reads Y's columns as rows
    {
      OP hi[4], lo[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        hi[ii] = cvt<OP>(x[ii]);
        lo[ii] = cvt<OP>(x[ii] - f32(hi[ii]));
      }
      using V4 = typename std::conditional<sizeof(OP) == 2, uint2, uint4>::type;   // four OP values
      const int o = (16 * nt + r16) * L::LDT + 16 * tw + 4 * q4;
      *reinterpret_cast<V4*>(sY + o) = *reinterpret_cast<const V4*>(hi);
      if constexpr (L::SPLIT) *reinterpret_cast<V4*>(sYl + o) = *reinterpret_cast<const V4*>(lo);
    }
  }
  __syncthreads();
  // ---- dA = -strict(T^T Y); dG = beta dA -> sA2; dbeta += rowsum(dA * G)
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int nt = 2 * hf + jj;
    f32x4 x = zero4();
#pragma unroll
    for (int k = 0; k < CH; k += 32)
      x = mma_ps(frag_row<OP>(sTT, L::LDT, 16 * tw + r16, k + kq), sfrag_pair<OP>(sY, sYl, L::LDT, 16 * nt + r16, k + kq), x);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int rr = 16 * tw + 4 * q4 + ii, cc = 16 * nt + r16;
      const float da = cc < rr ? -x[ii] : 0.f;
      dbeta[ii] += da * gGram[jj][ii];
      put_split(sA2h, sA2l, rr * L::LDQ + cc, sBeta[rr] * da);
    }
  }
  __syncthreads();

  // ---- per channel tile 2 jj + hf: gated products, then the assembly of dq, dk, dg.
  // PATH 0 (no 8-token span decaying past e^-STEEP_SPAN, see steep_block) uses one
  // reference row in the middle of each 16-row block and one product per step.
  // PATH 1 puts every decayed product e^{g_r - g_i} (i <= r) through reference rows
  // in the middle of 8-token groups (group_ref), split bf16 operands, with ch(R, C) =
  // e^{g_m(R) - g_m(C)} <= 1 the chain factor of groups C < R (1 for C = R, 0 above):
  // row side, tile a = tw:
  //   dq_g[r] = e^{g_r - g_m(R)} sum_i dAqk[r][i] k_i e^{g_m(C) - g_i} ch(R, C),  dkp_g likewise with dG;
  // column side, tile b = tw:
  //   dkm[i] = e^{g_m(C) - g_i} sum_r (dAqk[r][i] q_r + dG[r][i] k_r) e^{g_r - g_m(R)} ch(R, C).
  // The chain factor depends on the channel, so it goes into the channel-side operand:
  // each tile is two products, one per 8-token group of its output rows, accumulated
  // into one tile with the other group's rows of the token-side operand zeroed.  A
  // chain factor below CHAIN_MIN makes the wave form those channel-side values as one
  // exponential each instead.  One pass per channel tile: the pass's 32 channels (tiles
  // 2 jj and 2 jj + 1) get tables [channel][token] of the outer factors times q or k,
  // so the usual operand is a 16-byte LDS row read and each exponential is taken once
  // per element.
  O* dqo = reinterpret_cast<O*>(a.dq) + (size_t)ci.t0 * rk + (size_t)h * DK;
  O* dko = reinterpret_cast<O*>(a.dk_) + (size_t)ci.t0 * rk + (size_t)h * DK;
  O* dlo = reinterpret_cast<O*>(a.dla) + (size_t)ci.t0 * rk + (size_t)h * DK;
  float dgv[NKH][4];
  float khs[NKH];   // column sums over this lane's rows of dKh * Kh (for dg_C)
  float qdot[4] = {0.f, 0.f, 0.f, 0.f}, kdot[4] = {0.f, 0.f, 0.f, 0.f};   // q^.dq^, k^.dk^ (qk_norm)
  float* wDQ = qk_norm ? a.wsDQK + blk * (2 * CH * DK) : nullptr;
  float* wDK = qk_norm ? wDQ + CH * DK : nullptr;
  constexpr int TC = L::TC;
  static_assert(TC == 2 * 16 && NT == TC * (CH / 4), "table build: one thread per (channel, 4 tokens)");
  // chain factor of groups (R, C) for channel c: at most 1, zero above the diagonal
  auto chain = [&](int R, int C, int c) __attribute__((always_inline)) {
    const float e = __expf(sG[group_ref(R) * L::LDG + c] - sG[group_ref(C) * L::LDG + c]);
    return C < R ? e : (C == R ? 1.f : 0.f);
  };
  // 8 table values [channel cl][token t0 ..] times f
  auto scaled = [&](const float* tab, int cl, int t0, float f, float (&x)[8]) __attribute__((always_inline)) {
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(tab + cl * L::LDR + t0);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(tab + cl * L::LDR + t0 + 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      x[u] = v0[u] * f;
      x[u + 4] = v1[u] * f;
    }
  };
  // the tables of pass jj: one thread per (channel, 4 tokens)
  auto build_tables = [&](int jj, float* tq, float* tk, float* tkr) __attribute__((always_inline)) {
    {
      const int cl = tid % TC, r0 = 4 * (tid / TC);
      const int c = 32 * jj + cl;   // channel tiles 2 jj (cl < 16) and 2 jj + 1
      const float gm = sG[(PATH == 0 ? 16 * (r0 >> 4) + 8 : group_ref(r0 >> 3)) * L::LDG + c];
      float eq[4], ek[4], kr[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = r0 + u;
        const float g = sG[r * L::LDG + c];
        const float e = __expf(g - gm);
        const float kv = kn(r, c);
        eq[u] = qn(r, c) * e;
        ek[u] = kv * e;
        kr[u] = kv * __expf(gm - g);
      }
      *reinterpret_cast<f32x4*>(tq + cl * L::LDR + r0) = f32x4{eq[0], eq[1], eq[2], eq[3]};
      *reinterpret_cast<f32x4*>(tk + cl * L::LDR + r0) = f32x4{ek[0], ek[1], ek[2], ek[3]};
      *reinterpret_cast<f32x4*>(tkr + cl * L::LDR + r0) = f32x4{kr[0], kr[1], kr[2], kr[3]};
    }
  };
  build_tables(0, tQ, tK, tKR);
  __syncthreads();
  // (dk = 128 keeps the pass loop rolled: unrolled, it no longer fits the registers)
#pragma unroll(DK == 128 ? 1 : NKH)
  for (int jj = 0; jj < NKH; ++jj) {
    // with two table sets, pass jj reads set jj % 2 while it builds the next pass's
    // tables in the other (last read by pass jj - 1, which every wave has finished)
    const bool odd = L::TDB && (jj & 1);
    const float* cQ = odd ? tQ2 : tQ;
    const float* cK = odd ? tK2 : tK;
    const float* cKR = odd ? tKR2 : tKR;
    if constexpr (L::TDB) {
      if (jj + 1 < NKH) build_tables(jj + 1, odd ? tQ : tQ2, odd ? tK : tK2, odd ? tKR : tKR2);
    }
    const int cl = 16 * hf + r16, cc = 16 * (2 * jj + hf) + r16;
    const int hh = q4 >> 1;   // group 2 tw + hh holds this lane's output rows 16 tw + 4 q4 + ii
    f32x4 dqg = zero4(), dkpg = zero4(), dkm = zero4();
    if constexpr (PATH == 0) {   // reference rows in the middle of 16-row blocks, one product per step
      {
        const int ab = tw, kmax = 16 * (ab + 1);   // columns i < kmax can be nonzero
        const float gma = sG[(16 * ab + 8) * L::LDG + cc];
        for (int k = 0; k < kmax; k += 32) {
          const int i0 = k + kq, bb = i0 >> 4;
          const float f = i0 >= kmax ? 0.f : (bb == ab ? 1.f : __expf(gma - sG[(16 * bb + 8) * L::LDG + cc]));
          float xr[8];
          scaled(cKR, cl, i0, f, xr);
          const SFrag<SE> fr = sfrag_from<SE>(xr);
          dqg = mma_ss(sfrag_pair<SE>(sA1h, sA1l, L::LDQ, 16 * ab + r16, k + kq), fr, dqg);
          dkpg = mma_ss(sfrag_pair<SE>(sA2h, sA2l, L::LDQ, 16 * ab + r16, k + kq), fr, dkpg);
        }
  #pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float e = __expf(sG[(16 * ab + 4 * q4 + ii) * L::LDG + cc] - gma);
          dqg[ii] *= e;
          dkpg[ii] *= e;
        }
      }
      {
        const int b = tw;
        const float gmb = sG[(16 * b + 8) * L::LDG + cc];
        const bool useq = q4 < 2;
        const SE* aH = useq ? sA1h : sA2h;
        const SE* aL = useq ? sA1l : sA2l;
        const float* bT = useq ? cQ : cK;
        for (int ab = b; ab < 4; ++ab) {
          // block ab's reference factor goes into the channel-side operand, so the blocks
          // accumulate in the matrix core
          const int rbase = 16 * ab + 8 * (q4 & 1);
          const float f = ab == b ? 1.f : __expf(sG[(16 * ab + 8) * L::LDG + cc] - gmb);
          float xb[8];
          scaled(bT, cl, rbase, f, xb);
          dkm = mma_ss(sfrag_col_pair<SE>(aH, aL, L::LDQ, 16 * b + r16, rbase), sfrag_from<SE>(xb), dkm);
        }
  #pragma unroll
        for (int ii = 0; ii < 4; ++ii) dkm[ii] *= __expf(gmb - sG[(16 * b + 4 * q4 + ii) * L::LDG + cc]);
      }
    } else {
      {
        const int ab = tw, kmax = 16 * (ab + 1);   // columns i < kmax can be nonzero
        for (int k = 0; k < kmax; k += 32) {
          const int i0 = k + kq, C = i0 >> 3;   // this lane's 8 columns form group C
  #pragma unroll 1
          for (int g2 = 0; g2 < 2; ++g2) {
            const int R = 2 * ab + g2;
            const float f = chain(R, C, cc);   // zero past the diagonal block
            float xr[8];
            scaled(cKR, cl, i0, f, xr);
            if (__any(C < R && f < CHAIN_MIN) && C < R) {   // k_i e^{g_m(R) - g_i}, one exponential each
              const float gmr = sG[group_ref(R) * L::LDG + cc];
  #pragma unroll
              for (int u = 0; u < 8; ++u) xr[u] = kn(i0 + u, cc) * __expf(gmr - sG[(i0 + u) * L::LDG + cc]);
            }
            const SFrag<SE> fr = sfrag_from<SE>(xr);
            const bool mine = (r16 >> 3) == g2;   // this lane supplies row r16 of the tile
            dqg = mma_ss(sfrag_keep(sfrag_pair<SE>(sA1h, sA1l, L::LDQ, 16 * ab + r16, k + kq), mine), fr, dqg);
            dkpg = mma_ss(sfrag_keep(sfrag_pair<SE>(sA2h, sA2l, L::LDQ, 16 * ab + r16, k + kq), mine), fr, dkpg);
          }
        }
        const float gmr = sG[group_ref(2 * ab + hh) * L::LDG + cc];
  #pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float e = __expf(sG[(16 * ab + 4 * q4 + ii) * L::LDG + cc] - gmr);
          dqg[ii] *= e;
          dkpg[ii] *= e;
        }
      }
      {
        const int b = tw;
        // A[m = i][k = r'] : r' < 16 -> dAqk[16a + r'][i], r' >= 16 -> dG[16a + r' - 16][i];
        // B[k = r'][n] : decayed q rows of block a for r' < 16, decayed k rows for r' >= 16
        const bool useq = q4 < 2;
        const SE* aH = useq ? sA1h : sA2h;
        const SE* aL = useq ? sA1l : sA2l;
        const float* bT = useq ? cQ : cK;
        for (int ab = b; ab < 4; ++ab) {
          const int rbase = 16 * ab + 8 * (q4 & 1), R = rbase >> 3;   // this lane's 8 rows form group R
  #pragma unroll 1
          for (int g2 = 0; g2 < 2; ++g2) {
            const int C = 2 * b + g2;
            const float f = chain(R, C, cc);   // zero for rows above the output group
            float xb[8];
            scaled(bT, cl, rbase, f, xb);
            if (__any(C < R && f < CHAIN_MIN) && C < R) {   // w_r e^{g_r - g_m(C)}, one exponential each
              const float gmc = sG[group_ref(C) * L::LDG + cc];
  #pragma unroll
              for (int u = 0; u < 8; ++u)
                xb[u] = (useq ? qn(rbase + u, cc) : kn(rbase + u, cc)) * __expf(sG[(rbase + u) * L::LDG + cc] - gmc);
            }
            dkm = mma_ss(sfrag_keep(sfrag_col_pair<SE>(aH, aL, L::LDQ, 16 * b + r16, rbase), (r16 >> 3) == g2),
                         sfrag_from<SE>(xb), dkm);
          }
        }
        const float gmc = sG[group_ref(2 * b + hh) * L::LDG + cc];
  #pragma unroll
        for (int ii = 0; ii < 4; ++ii) dkm[ii] *= __expf(gmc - sG[(16 * b + 4 * q4 + ii) * L::LDG + cc]);
      }
    }
    // assembly (rows 16tw + 4q4 + ii)
    {
      khs[jj] = 0.f;
      const float gl = sG[(CH - 1) * L::LDG + cc];
      f32x4 vq, vk;   // this lane's dq, dk tile values (rows 4 q4 + ii)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int rr = 16 * tw + 4 * q4 + ii;
        const float g = sG[rr * L::LDG + cc];
        const float eg = __expf(g);
        const float kv = kn(rr, cc), qv = qn(rr, cc);
        const float dq = eg * scale * accQ[jj][ii] + dqg[ii];
        const float dkp = eg * sBeta[rr] * tdw[jj][ii] + dkpg[ii];
        const float dkmv = dkm[ii];
        const float dkh = __expf(gl - g) * accK[jj][ii];
        dgv[jj][ii] = dq * qv + (dkp - dkmv - dkh) * kv;
        khs[jj] += dkh * kv;
        const float dkt = dkp + dkmv + dkh;
        vq[ii] = dq;
        vk[ii] = dkt;
        if constexpr (qk_norm) {
          qdot[ii] += qv * dq;
          kdot[ii] += kv * dkt;
        }
      }
      // stores after a quad transpose: this lane holds row 16 tw + 4 q4 + (r16 & 3),
      // columns cc - (r16 & 3) .. + 3
      vq = quad_transpose(vq);
      vk = quad_transpose(vk);
      const int rt = 16 * tw + 4 * q4 + (r16 & 3), ct = cc - (r16 & 3);
      if constexpr (qk_norm) {   // gradients of the normalised rows; the chain rule follows below
        *reinterpret_cast<f32x4*>(wDQ + rt * DK + ct) = vq;
        *reinterpret_cast<f32x4*>(wDK + rt * DK + ct) = vk;
      } else if (rt < len) {
        store4<O>(dqo + (size_t)rt * rk + ct, gs_inv * vq[0], gs_inv * vq[1], gs_inv * vq[2], gs_inv * vq[3]);
        store4<O>(dko + (size_t)rt * rk + ct, gs_inv * vk[0], gs_inv * vk[1], gs_inv * vk[2], gs_inv * vk[3]);
      }
    }
    if (jj + 1 < NKH) {
      if constexpr (!L::TDB) {   // one set: the pass's table reads end before the next build
        __syncthreads();
        build_tables(jj + 1, tQ, tK, tKR);
      }
      __syncthreads();   // the next pass's tables are complete
    }
  }
  // the raw gate values of the rows this thread finishes in the reverse sum below (channel
  // tid % DK, rows of part tid / DK), all issued now so that their latency overlaps the
  // reductions; rows past the chunk read the last row and are not stored
  E xlr[RPS];
  {
    const int c = tid % DK, s = tid / DK;
#pragma unroll
    for (int u = 0; u < RPS; ++u) xlr[u] = lh[(size_t)min(s * RPS + u, len - 1) * rk + c];
  }
  // dbeta partials: reduce over the 16 column lanes; halves meet in LDS
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const float p = lane_sum16(dbeta[ii]);
    if (r16 == 0) sDbp[hf * CH + 16 * tw + 4 * q4 + ii] = p;
  }
  if constexpr (qk_norm) {   // row dots: reduce over the 16 column lanes; halves meet in LDS
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const float pq = lane_sum16(qdot[ii]), pk = lane_sum16(kdot[ii]);
      if (r16 == 0) {
        sDot[hf * CH + 16 * tw + 4 * q4 + ii] = pq;
        sDot[2 * CH + hf * CH + 16 * tw + 4 * q4 + ii] = pk;
      }
    }
    __threadfence_block();   // the workspace rows of dq^, dk^ are read by other threads below
  }
  __syncthreads();  // all reads of g are done before dg overwrites it
#pragma unroll
  for (int jj = 0; jj < NKH; ++jj) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) sG[(16 * tw + 4 * q4 + ii) * L::LDG + 16 * (2 * jj + hf) + r16] = dgv[jj][ii];
    float p = khs[jj];
    p += __shfl_xor(p, 16);
    p += __shfl_xor(p, 32);
    if (q4 == 0) sRed[tw * DK + 16 * (2 * jj + hf) + r16] = p;
  }
  __syncthreads();
  if (tid < CH) {
    const int rr = tid;
    if (rr < len)
      reinterpret_cast<O*>(a.dbeta)[((size_t)ci.t0 + rr) * H + h] =
          cvt<O>(gs_inv * ((sDbp[rr] + sDbp[CH + rr]) + (sBv[rr] + sBv[CH + rr])));
  } else if (tid >= 64 && tid < 64 + DK) {
    // dg_C: the last row collects sum_r dKh * Kh and dGamma_C * Gamma_C
    const int c = tid - 64;
    const float s = (sRed[c] + sRed[DK + c]) + (sRed[2 * DK + c] + sRed[3 * DK + c]);
    sG[(CH - 1) * L::LDG + c] += s + sDGam[c] * gam_c;
  }
  __syncthreads();
  // reverse cumulative sum over rows -> dlog_alpha
  {
    const int c = tid % DK, s = tid / DK;
    float acc = 0.f;
#pragma unroll
    for (int rr = (s + 1) * RPS - 1; rr >= s * RPS; --rr) acc += sG[rr * L::LDG + c];
    sRed[s * DK + c] = acc;
  }
  __syncthreads();
  {
    const int c = tid % DK, s = tid / DK;
    float acc = 0.f;
    for (int s2 = s + 1; s2 < NSPLIT; ++s2) acc += sRed[s2 * DK + c];
#pragma unroll
    for (int u = RPS - 1; u >= 0; --u) {
      const int rr = s * RPS + u;
      acc += sG[rr * L::LDG + c];
      if (rr < len) {
        // through the gate's map and the floor of log alpha (flat below it)
        const float x = f32(xlr[u]);
        const float d = gs_inv * (a.gate_ls ? acc * sigmoid_neg(x) : acc);
        dlo[(size_t)rr * rk + c] = cvt<O>(above_floor(a.gate_ls ? logsigmoid(x) : x) ? d : 0.f);
      }
    }
  }
  if constexpr (qk_norm) {
    // d x = (1/|x|) (d x^ - x^ (x^ . d x^)) for the raw q and k rows (unrolled, so the
    // loads of dq^, dk^ are all in flight together)
#pragma unroll
    for (int o = tid; o < 2 * CH * DK / 4; o += NT) {
      const int which = o / (CH * DK / 4), e = 4 * (o % (CH * DK / 4));
      const int rr = e / DK, c0 = e % DK;
      if (rr >= len) continue;
      const float* src = which ? wDK : wDQ;
      const E* xh = which ? sK : sQ;
      const f32x4 g = *reinterpret_cast<const f32x4*>(src + rr * DK + c0);
      const float dot = sDot[2 * CH * which + rr] + sDot[2 * CH * which + CH + rr];
      const float sc = sNrm[CH * which + rr];
      O* dst = (which ? dko : dqo) + (size_t)rr * rk + c0;
      float y[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) y[u] = gs_inv * (sc * (g[u] - f32(xh[rr * L::LDK + c0 + u]) * sc * dot));
      store4<O>(dst, y[0], y[1], y[2], y[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV, int DVS, bool LOCAL = false>
static hipError_t launch_rev(const Args& a, hipStream_t st) {
  constexpr int NSL = DV / DVS;
  const int grid = (a.N * a.H + 7) / 8 * 8 * NSL;
  KDA_TIMED(LOCAL ? "kda_seg_rev_local" : "kda_state_bwd_revpass", st,
            hipLaunchKernelGGL((kda_state_rev<E, DK, DV, DVS, LOCAL>), dim3(grid), dim3(512), 0, st, a));
  return hipGetLastError();
}

template <typename E, int DK, int DV, bool LOCAL = false>
static hipError_t launch_rev_auto(const Args& a, hipStream_t st) {
  if (a.N * a.H == 0) return hipSuccess;
  if constexpr (sizeof(E) == 2) {
    if (pick_dvs(a.N * a.H, DV) == 64) return launch_rev<E, DK, DV, 64, LOCAL>(a, st);
    return launch_rev<E, DK, DV, 16, LOCAL>(a, st);
  } else {
    return launch_rev<E, DK, DV, 32, LOCAL>(a, st);
  }
}

// Segmented reverse pass (long sequences cut into the forward's stretches): each
// stretch runs from dS' = 0 (in parallel), a reverse scan per (sequence, head)
// with the transposed stretch transfers M^T the forward left in seg_m gives each
// stretch the true gradient of the state leaving it, and the ordinary reverse
// pass then runs every stretch from that gradient at once.
template <typename E, int DK, int DV>
static hipError_t launch_segmented_rev(const Args& a, hipStream_t st) {
  hipError_t e = launch_segment_map(a, st);   // the same stretches as the forward (idempotent)
  if (e != hipSuccess) return e;
  Args av = a;   // the stretches as sequences of their own
  av.N = a.N * a.segs;
  av.seq_chunk0 = a.vsc0;
  av.seq_order = a.vord;
  Args al = av;
  al.dfinal = nullptr;
  al.dinit = a.seg_loc;   // gradient entering each stretch, from zero
  if ((e = launch_rev_auto<E, DK, DV, true>(al, st)) != hipSuccess) return e;
  if ((e = launch_segment_rscan<DK, DV>(a, st)) != hipSuccess) return e;   // seg_in, d_init_state
  Args af = av;
  af.dfinal = a.seg_in;
  af.dfinal_scaled = 1;
  af.dinit = nullptr;
  return launch_rev_auto<E, DK, DV>(af, st);
}

// `saved`: the workspace already holds the forward intermediates (kda_fwd with
// KDA_FLAG_SAVE_FOR_BACKWARD on the same inputs), so the front half is skipped.
template <typename E, typename O, int DK, int DV>
hipError_t launch_bwd(const Args& a, hipStream_t st, bool saved) {
  hipError_t e = hipSuccess;
  if (!saved) {
    e = launch_bwd_front<E, DK, DV>(a, st);
    if (e != hipSuccess) return e;
  }
  if (a.gscale && (e = launch_grad_scale(a, st)) != hipSuccess) return e;
  e = a.segs > 1 ? launch_segmented_rev<E, DK, DV>(a, st) : launch_rev_auto<E, DK, DV>(a, st);
  if (e != hipSuccess) return e;
  if (a.max_chunks > 0) {
    // bf16: the usual chunk-heads, then the ones the prep flagged as steep; the fp32
    // prep flags every chunk-head
#define KDA_BWDC(QKN)                                                                                      \
  do {                                                                                                     \
    if constexpr (sizeof(E) == 2)                                                                          \
      KDA_TIMED("kda_bwd_chunk", st, hipLaunchKernelGGL((kda_bwd_chunk<E, O, DK, DV, QKN, 0>),             \
                                                        dim3(a.max_chunks, a.H), dim3(512), 0, st, a));    \
    KDA_TIMED(sizeof(E) == 2 ? "kda_bwd_chunk_steep" : "kda_bwd_chunk", st,                                \
              hipLaunchKernelGGL((kda_bwd_chunk<E, O, DK, DV, QKN, 1>), dim3(a.max_chunks, a.H), dim3(512), \
                                 0, st, a));                                                               \
  } while (0)
    if (a.qk_norm)
      KDA_BWDC(true);
    else
      KDA_BWDC(false);
#undef KDA_BWDC
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

#define KDA_INST(E, O, DK, DV) template hipError_t launch_bwd<E, O, DK, DV>(const Args&, hipStream_t, bool);
KDA_INST(bf16, float, 64, 64)
KDA_INST(bf16, float, 64, 128)
KDA_INST(bf16, float, 128, 64)
KDA_INST(bf16, float, 128, 128)
KDA_INST(bf16, bf16, 64, 64)
KDA_INST(bf16, bf16, 64, 128)
KDA_INST(bf16, bf16, 128, 64)
KDA_INST(bf16, bf16, 128, 128)
KDA_INST(float, float, 64, 64)
KDA_INST(float, float, 64, 128)
#undef KDA_INST

}  // namespace kda
