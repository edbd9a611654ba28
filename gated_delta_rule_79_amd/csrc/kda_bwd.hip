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
//   kda_bwd_dv      : chunk-parallel contractions over the value dimension.
//   kda_bwd_dk      : chunk-parallel contractions over tokens, gated products,
//                     and the assembly of dq, dk, dlog_alpha, dbeta.
// The gated products never form K- = K/Gamma: they use the same per-block
// reference rows as the forward's decayed Gram blocks.
#include "kda_internal.hpp"

namespace kda {

template <typename E, int DK, int DV>
hipError_t launch_bwd_front(const Args& a, hipStream_t st);

// ---------------------------------------------------------------------------
// reverse sequential pass
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV, int DVS>
struct RevLds {
  using OP = typename OpOf<E>::T;
  static constexpr int P = PADE<OP>;
  static constexpr int LDK = DK + P;
  static constexpr int LDT = CH + P;
  static constexpr int LDF = DK + 4;
  static constexpr size_t AQK = 0;                                          // OP    [CH][LDT]
  static constexpr size_t KHF = AQK + (size_t)CH * LDT * sizeof(OP);        // float [CH][LDF]
  static constexpr size_t QT = KHF + (size_t)CH * LDF * 4;                  // OP    [CH][LDK]
  static constexpr size_t W = QT + (size_t)CH * LDK * sizeof(OP);           // OP    [CH][LDK]
  static constexpr size_t GAM = W + (size_t)CH * LDK * sizeof(OP);          // float [DK]
  static constexpr size_t DOT = GAM + (size_t)DK * 4;                       // OP    [DVS][LDT]  dO^T slice
  static constexpr size_t DSH = DOT + (size_t)DVS * LDT * sizeof(OP);       // OP    [DVS][LDK]  dS'^T split
  static constexpr size_t DSL = DSH + (size_t)DVS * LDK * sizeof(OP);
  static constexpr size_t DUH = DSL + (size_t)DVS * LDK * sizeof(OP);       // OP    [DVS][LDT]  dU^T split
  static constexpr size_t DUL = DUH + (size_t)DVS * LDT * sizeof(OP);
  static constexpr size_t BYTES = DUL + (size_t)DVS * LDT * sizeof(OP);
  static_assert(BYTES <= 163840, "reverse pass LDS");
};

template <typename E, int DK, int DV, int DVS>
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
  const int seq = unit / a.H, h = unit % a.H, H = a.H;
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
  float* sKhF = reinterpret_cast<float*>(smem + L::KHF);
  OP* sQt = reinterpret_cast<OP*>(smem + L::QT);
  OP* sW = reinterpret_cast<OP*>(smem + L::W);
  float* sGam = reinterpret_cast<float*>(smem + L::GAM);
  OP* sDOT = reinterpret_cast<OP*>(smem + L::DOT);
  OP* sDSh = reinterpret_cast<OP*>(smem + L::DSH);
  OP* sDSl = reinterpret_cast<OP*>(smem + L::DSL);
  OP* sDUh = reinterpret_cast<OP*>(smem + L::DUH);
  OP* sDUl = reinterpret_cast<OP*>(smem + L::DUL);

  const OP* gAqk = reinterpret_cast<const OP*>(a.wsAqk);
  const float* gKhF = a.wsKhF;
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

  f32x4 dS[SPW];
  const size_t st_off = ((size_t)seq * H + h) * DK * DV;
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int t = w + 8 * i, mt = t % MTS, nt = t / MTS;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int ch = 16 * mt + 4 * q4 + ii, col = n0 + 16 * nt + r16;
      dS[i][ii] = (gDFin && t < NST) ? gDFin[st_off + (size_t)ch * DV + col] : 0.f;
    }
  }

  // dO slice: 64 token rows x DVS columns of the input, rows past the chunk zeroed
  constexpr int EPV = 16 / (int)sizeof(E), VPR = DVS / EPV, NVO = CH * VPR;
  struct Stage {
    TileCopy<OP, CH, CH, NT> aqk;
    TileCopy<float, CH, DK, NT> khf;
    TileCopy<OP, CH, DK, NT> qt;
    TileCopy<OP, CH, DK, NT> w;
    TileCopy<float, 1, DK, NT> gam;
    u32x4 dov;  // one 16-byte piece of the dO slice (threads < NVO)
    int dolen;
  };
  static_assert(NVO <= NT, "dO slice staging");
  Stage st0, st1;
  auto blk_of = [&](int n) { return (size_t)(c0 + n) * H + h; };
  auto stage_load = [&](Stage& p, int n) __attribute__((always_inline)) {
    const size_t b = blk_of(n);
    p.aqk.load(gAqk + b * WB::AQK, CH);
    p.khf.load(gKhF + b * WB::KHF, DK);
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
    p.khf.store(sKhF, L::LDF);
    p.qt.store(sQt, L::LDK);
    p.w.store(sW, L::LDK);
    p.gam.store(sGam, DK);
    if (tid < NVO) {
      const int row = tid / VPR, cv = tid % VPR;
      const bool ok = row < p.dolen;
      const E* e = reinterpret_cast<const E*>(&p.dov);
#pragma unroll
      for (int i = 0; i < EPV; ++i) sDOT[(cv * EPV + i) * L::LDT + row] = cvt<OP>(ok ? f32(e[i]) : 0.f);
    }
  };

  auto chunk = [&](int n, Stage& ld, const Stage& nx) __attribute__((always_inline)) {
    stage_load(ld, max(n - 2, 0));
    // dS' (gradient of the state leaving chunk n) -> LDS split, and -> workspace fp32
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = w + 8 * i, mt = t % MTS, nt = t / MTS;
      if (t < NST) {
        const int off = (16 * nt + r16) * L::LDK + 16 * mt + 4 * q4;
        store4_split<OP>(sDSh + off, sDSl + off, dS[i][0], dS[i][1], dS[i][2], dS[i][3]);
        float* dst = gdS + blk_of(n) * WB::DS + (size_t)(n0 + 16 * nt + r16) * DK + 16 * mt + 4 * q4;
        *reinterpret_cast<f32x4*>(dst) = dS[i];
      }
    }
    __syncthreads();

    if (w < 4) {
      // dU (token tile w) = scale Aqk^T dO + Kh dS'
#pragma unroll
      for (int nt = 0; nt < NTS; ++nt) {
        f32x4 x1 = zero4(), x2 = zero4();
#pragma unroll
        for (int k = 0; k < CH; k += 32)
          x1 = mma(frag_col<OP>(sAqk, L::LDT, 16 * w + r16, k + 8 * q4),
                   frag_row<OP>(sDOT, L::LDT, 16 * nt + r16, k + 8 * q4), x1);
#pragma unroll
        for (int k = 0; k < DK; k += 32)
          x2 = mma_ss(sfrag_row<OP>(sKhF, L::LDF, 16 * w + r16, k + 8 * q4),
                      sfrag_pair<OP>(sDSh, sDSl, L::LDK, 16 * nt + r16, k + 8 * q4), x2);
        const f32x4 du = scale * x1 + x2;
        const int off = (16 * nt + r16) * L::LDT + 16 * w + 4 * q4;
        store4_split<OP>(sDUh + off, sDUl + off, du[0], du[1], du[2], du[3]);
        float* dst = gdU + blk_of(n) * WB::DU + (size_t)(n0 + 16 * nt + r16) * CH + 16 * w + 4 * q4;
        *reinterpret_cast<f32x4*>(dst) = du;
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
          qd[i] = mma(frag_col<OP>(sQt, L::LDK, 16 * mt + r16, k + 8 * q4),
                      frag_row<OP>(sDOT, L::LDT, 16 * nt + r16, k + 8 * q4), qd[i]);
      }
    }
    __syncthreads();
    // dS = Gamma_C dS' + scale Qt^T dO - W^T dU
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = w + 8 * i, mt = t % MTS, nt = t / MTS;
      if (t < NST) {
        f32x4 x = zero4();
#pragma unroll
        for (int k = 0; k < CH; k += 32)
          x = mma_ps(frag_col<OP>(sW, L::LDK, 16 * mt + r16, k + 8 * q4),
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
    stage_load(st0, nch - 1);
    stage_store(st0);
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
          gDInit[st_off + (size_t)ch * DV + col] = dS[i][ii];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// chunk-parallel contractions over the value dimension
// ---------------------------------------------------------------------------
// Wave w owns token rows 16w..16w+15 of every output; the value dimension is
// walked in quarters of 32 columns so the working set fits in LDS.
template <typename E, int DK, int DV>
struct DvLds {
  using OP = typename OpOf<E>::T;
  static constexpr int P = PADE<OP>;
  static constexpr int QC = 32;             // value columns per pass
  static constexpr int LDK = DK + P;
  static constexpr int LDT = CH + P;
  static constexpr int LDQ = QC + P;
  static constexpr size_t T = 0;                                           // OP [CH][LDT]
  static constexpr size_t S = T + (size_t)CH * LDT * sizeof(OP);           // OP [QC][LDK]   S^T quarter
  static constexpr size_t DSH = S + (size_t)QC * LDK * sizeof(OP);         // OP [QC][LDK]   dS'^T split
  static constexpr size_t DSL = DSH + (size_t)QC * LDK * sizeof(OP);
  static constexpr size_t UH = DSL + (size_t)QC * LDK * sizeof(OP);        // OP [QC][LDT]   U^T split
  static constexpr size_t UL = UH + (size_t)QC * LDT * sizeof(OP);
  static constexpr size_t DUH = UL + (size_t)QC * LDT * sizeof(OP);        // OP [QC][LDT]   dU^T split
  static constexpr size_t DUL = DUH + (size_t)QC * LDT * sizeof(OP);
  static constexpr size_t DO = DUL + (size_t)QC * LDT * sizeof(OP);        // OP [CH][LDQ]   dO quarter
  static constexpr size_t V = DO + (size_t)CH * LDQ * sizeof(OP);          // OP [CH][LDQ]   V quarter
  static constexpr size_t BETA = V + (size_t)CH * LDQ * sizeof(OP);        // float [CH]
  static constexpr size_t GAMP = BETA + CH * 4;                            // float [256] partial rowsums
  static constexpr size_t BYTES = GAMP + 256 * 4;
  static_assert(BYTES <= 163840, "dv kernel LDS");
};

template <typename E, typename O, int DK, int DV>
__global__ __launch_bounds__(256) void kda_bwd_dv(const Args a) {
  using L = DvLds<E, DK, DV>;
  using OP = typename L::OP;
  using WB = WsBlock<E, DK, DV>;
  constexpr int NT = 256, QC = L::QC, NQ = DV / QC;
  constexpr int NKT = DK / 16;   // channel tiles
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  const int j = blockIdx.x, h = blockIdx.y, H = a.H;
  const ChunkInfo ci = a.chunks[j];
  if (ci.len <= 0) return;
  const int len = ci.len;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), r16 = l & 15, q4 = l >> 4;
  const size_t blk = (size_t)j * H + h;
  const size_t rv = (size_t)H * DV;

  OP* sT = reinterpret_cast<OP*>(smem + L::T);
  OP* sS = reinterpret_cast<OP*>(smem + L::S);
  OP* sDSh = reinterpret_cast<OP*>(smem + L::DSH);
  OP* sDSl = reinterpret_cast<OP*>(smem + L::DSL);
  OP* sUh = reinterpret_cast<OP*>(smem + L::UH);
  OP* sUl = reinterpret_cast<OP*>(smem + L::UL);
  OP* sDUh = reinterpret_cast<OP*>(smem + L::DUH);
  OP* sDUl = reinterpret_cast<OP*>(smem + L::DUL);
  OP* sDO = reinterpret_cast<OP*>(smem + L::DO);
  OP* sV = reinterpret_cast<OP*>(smem + L::V);
  float* sBeta = reinterpret_cast<float*>(smem + L::BETA);
  float* sGamP = reinterpret_cast<float*>(smem + L::GAMP);

  const E* gV = reinterpret_cast<const E*>(a.v) + (size_t)ci.t0 * rv + (size_t)h * DV;
  const E* gDO = reinterpret_cast<const E*>(a.dout) + (size_t)ci.t0 * rv + (size_t)h * DV;
  const E* gB = reinterpret_cast<const E*>(a.beta) + (size_t)ci.t0 * H + h;
  const OP* gS = reinterpret_cast<const OP*>(a.wsS) + blk * WB::S;
  const float* gdS = a.wsdS + blk * WB::DS;
  const float* gU = a.wsU + blk * WB::U;
  const float* gdU = a.wsdU + blk * WB::DU;
  const float* gT = reinterpret_cast<const float*>(a.wsT) + blk * WB::TT;
  O* gdV = reinterpret_cast<O*>(a.dv_) + (size_t)ci.t0 * rv + (size_t)h * DV;

  for (int o = tid; o < CH * CH; o += NT) sT[(o / CH) * L::LDT + o % CH] = cvt<OP>(gT[o]);
  if (tid < CH) sBeta[tid] = tid < len ? f32(gB[(size_t)tid * H]) : 0.f;

  f32x4 accA[4], accQ[NKT], accK[NKT], accW[NKT], accT[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) accA[i] = accT[i] = zero4();
#pragma unroll
  for (int i = 0; i < NKT; ++i) accQ[i] = accK[i] = accW[i] = zero4();
  float bv[4] = {0.f, 0.f, 0.f, 0.f};   // rowsum(V * T^T dU) partials for rows 16w + 4q4 + ii (lane r16 == 0)
  float gp = 0.f;                       // rowsum(dS' * S) partial for channel tid % DK

  for (int qq = 0; qq < NQ; ++qq) {
    const int cq = qq * QC;
    __syncthreads();  // previous quarter's LDS reads are done
    // S^T and dS'^T quarter: rows cq..cq+QC of [DV][DK]
    {
      constexpr int VPR = DK / 8;
      for (int v = tid; v < QC * VPR; v += NT) {
        const int row = v / VPR, c0 = (v % VPR) * 8;
        float s8[8];
        load8<OP>(gS + (size_t)(cq + row) * DK + c0, true, s8);
        store4<OP>(sS + row * L::LDK + c0, s8[0], s8[1], s8[2], s8[3]);
        store4<OP>(sS + row * L::LDK + c0 + 4, s8[4], s8[5], s8[6], s8[7]);
        const float* src = gdS + (size_t)(cq + row) * DK + c0;
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(src);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(src + 4);
        store4_split<OP>(sDSh + row * L::LDK + c0, sDSl + row * L::LDK + c0, d0[0], d0[1], d0[2], d0[3]);
        store4_split<OP>(sDSh + row * L::LDK + c0 + 4, sDSl + row * L::LDK + c0 + 4, d1[0], d1[1], d1[2], d1[3]);
      }
      // U^T, dU^T quarter: rows cq..cq+QC of [DV][CH]
      constexpr int VPT = CH / 4;
      for (int v = tid; v < QC * VPT; v += NT) {
        const int row = v / VPT, c0 = (v % VPT) * 4;
        const f32x4 u = *reinterpret_cast<const f32x4*>(gU + (size_t)(cq + row) * CH + c0);
        const f32x4 du = *reinterpret_cast<const f32x4*>(gdU + (size_t)(cq + row) * CH + c0);
        store4_split<OP>(sUh + row * L::LDT + c0, sUl + row * L::LDT + c0, u[0], u[1], u[2], u[3]);
        store4_split<OP>(sDUh + row * L::LDT + c0, sDUl + row * L::LDT + c0, du[0], du[1], du[2], du[3]);
      }
      // dO and V quarters, token-major, rows past the chunk zeroed
      constexpr int VPQ = QC / 8;
      for (int v = tid; v < CH * VPQ; v += NT) {
        const int row = v / VPQ, c0 = (v % VPQ) * 8;
        float x[8], y[8];
        load8<E>(gDO + (size_t)row * rv + cq + c0, row < len, x);
        load8<E>(gV + (size_t)row * rv + cq + c0, row < len, y);
        store4<OP>(sDO + row * L::LDQ + c0, x[0], x[1], x[2], x[3]);
        store4<OP>(sDO + row * L::LDQ + c0 + 4, x[4], x[5], x[6], x[7]);
        store4<OP>(sV + row * L::LDQ + c0, y[0], y[1], y[2], y[3]);
        store4<OP>(sV + row * L::LDQ + c0 + 4, y[4], y[5], y[6], y[7]);
      }
    }
    __syncthreads();
    // rowsum over values of dS' * S (channel c, half of the quarter's columns)
    {
      const int c = tid % DK, part = tid / DK;  // NT / DK parts
      constexpr int NPART = NT / DK, CPP = QC / NPART;
      for (int col = part * CPP; col < (part + 1) * CPP; ++col) {
        const int o = col * L::LDK + c;
        // the low half exists only for 2-byte operands (store4_split leaves it unwritten for fp32)
        const float ds = sizeof(OP) == 2 ? f32(sDSh[o]) + f32(sDSl[o]) : f32(sDSh[o]);
        gp += ds * f32(sS[o]);
      }
    }
    const int kq = 8 * q4;
    const Frag<OP> fdo = frag_row<OP>(sDO, L::LDQ, 16 * w + r16, kq);        // dO rows of tile w
    const SFrag<OP> fdu = sfrag_col_pair<OP>(sDUh, sDUl, L::LDT, 16 * w + r16, kq);   // dU rows of tile w
    const SFrag<OP> fu = sfrag_col_pair<OP>(sUh, sUl, L::LDT, 16 * w + r16, kq);      // U rows of tile w
    // dAqk += dO U^T ; dT_U += dU V^T
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      accA[nt] = mma_ps(fdo, sfrag_col_pair<OP>(sUh, sUl, L::LDT, 16 * nt + r16, kq), accA[nt]);
      accT[nt] = mma_sp(fdu, frag_row<OP>(sV, L::LDQ, 16 * nt + r16, kq), accT[nt]);
    }
    // dQS += dO S^T ; dKh += U dS'^T ; dW += dU S^T
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) {
      const Frag<OP> fs = frag_col<OP>(sS, L::LDK, 16 * nt + r16, kq);
      accQ[nt] = mma(fdo, fs, accQ[nt]);
      accW[nt] = mma_sp(fdu, fs, accW[nt]);
      accK[nt] = mma_ss(fu, sfrag_col_pair<OP>(sDSh, sDSl, L::LDK, 16 * nt + r16, kq), accK[nt]);
    }
    // T^T dU for token tile w and the quarter's columns -> dV, and rowsum(V * T^T dU)
#pragma unroll
    for (int nt = 0; nt < QC / 16; ++nt) {
      f32x4 x = zero4();
#pragma unroll
      for (int k = 0; k < CH; k += 32)
        x = mma_ps(frag_col<OP>(sT, L::LDT, 16 * w + r16, k + kq),
                   sfrag_pair<OP>(sDUh, sDUl, L::LDT, 16 * nt + r16, k + kq), x);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 16 * w + 4 * q4 + ii, col = 16 * nt + r16;
        float p = f32(sV[r * L::LDQ + col]) * x[ii];
        p += __shfl_xor(p, 1);
        p += __shfl_xor(p, 2);
        p += __shfl_xor(p, 4);
        p += __shfl_xor(p, 8);
        bv[ii] += p;
        if (r < len) gdV[(size_t)r * rv + cq + col] = cvt<O>(sBeta[r] * x[ii]);
      }
    }
  }

  // outputs of this kernel (fp32 workspace), rows 16w + 4q4 + ii
  const float scale = a.scale;
  float* wA = a.wsdAqk + blk * WB::DAQK;
  float* wTU = a.wsdTU + blk * WB::DTU;
  float* wQ = a.wsdQS + blk * WB::DQS;
  float* wK = a.wsdKh + blk * WB::DKH;
  float* wW = a.wsdW + blk * WB::DW;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int r = 16 * w + 4 * q4 + ii;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int c = 16 * nt + r16;
      wA[r * CH + c] = c <= r ? scale * accA[nt][ii] : 0.f;
      wTU[r * CH + c] = accT[nt][ii] * sBeta[c];
    }
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) {
      const int c = 16 * nt + r16;
      wQ[r * DK + c] = scale * accQ[nt][ii];
      wK[r * DK + c] = accK[nt][ii];
      wW[r * DK + c] = -accW[nt][ii];
    }
    if (r16 == 0) a.wsdBv[blk * WB::DBV + r] = bv[ii];
  }
  sGamP[tid] = gp;  // part tid / DK of channel tid % DK
  __syncthreads();
  if (tid < DK) {
    float s = 0.f;
    for (int p = 0; p < NT / DK; ++p) s += sGamP[p * DK + tid];
    a.wsdGam[blk * WB::DGAM + tid] = s;
  }
}

// ---------------------------------------------------------------------------
// chunk-parallel contractions over tokens, gated products and assembly
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV>
struct DkLds {
  using OP = typename OpOf<E>::T;
  static constexpr int PE = PADE<E>, PO = PADE<OP>;
  static constexpr int LDG = DK + 4;
  static constexpr int LDK = DK + PE;   // E rows
  static constexpr int LDO = DK + PO;   // OP rows
  static constexpr int LDT = CH + PO;
  static constexpr int LDA = CH + 4;
  static constexpr size_t G = 0;                                             // float [CH][LDG]  g, later dg
  static constexpr size_t K = G + (size_t)CH * LDG * 4;                      // E     [CH][LDK]
  static constexpr size_t Q = K + (size_t)CH * LDK * sizeof(E);              // E     [CH][LDK]
  static constexpr size_t T = Q + (size_t)CH * LDK * sizeof(E);              // OP    [CH][LDT]
  static constexpr size_t A1 = T + (size_t)CH * LDT * sizeof(OP);            // float [CH][LDA]  dAqk
  static constexpr size_t A2 = A1 + (size_t)CH * LDA * 4;                    // float [CH][LDA]  dT, then dG
  static constexpr size_t DW = A2 + (size_t)CH * LDA * 4;                    // OP    [CH][LDO]  dW, then Y
  static constexpr size_t KP = DW + (size_t)CH * LDO * sizeof(OP);           // OP    [CH][LDO]  K+
  static constexpr size_t BETA = KP + (size_t)CH * LDO * sizeof(OP);         // float [CH]
  static constexpr size_t RED = BETA + CH * 4;                               // float [4][DK] reductions
  static constexpr size_t BYTES = RED + 4 * DK * 4;
  static constexpr size_t Y = DW;                                            // OP [CH][LDT] (after dW is dead)
  static_assert(BYTES <= 163840, "dk kernel LDS");
};

template <typename E, typename O, int DK, int DV>
__global__ __launch_bounds__(256) void kda_bwd_dk(const Args a) {
  using L = DkLds<E, DK, DV>;
  using OP = typename L::OP;
  using WB = WsBlock<E, DK, DV>;
  using SE = typename std::conditional<sizeof(E) == 4, float, bf16>::type;   // gated products: split bf16
  constexpr int NT = 256, NKT = DK / 16;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  const int j = blockIdx.x, h = blockIdx.y, H = a.H;
  const ChunkInfo ci = a.chunks[j];
  if (ci.len <= 0) return;
  const int len = ci.len;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), r16 = l & 15, q4 = l >> 4;
  const size_t blk = (size_t)j * H + h;
  const size_t rk = (size_t)H * DK;

  float* sG = reinterpret_cast<float*>(smem + L::G);
  E* sK = reinterpret_cast<E*>(smem + L::K);
  E* sQ = reinterpret_cast<E*>(smem + L::Q);
  OP* sT = reinterpret_cast<OP*>(smem + L::T);
  float* sA1 = reinterpret_cast<float*>(smem + L::A1);
  float* sA2 = reinterpret_cast<float*>(smem + L::A2);
  OP* sDW = reinterpret_cast<OP*>(smem + L::DW);
  OP* sKp = reinterpret_cast<OP*>(smem + L::KP);
  OP* sY = reinterpret_cast<OP*>(smem + L::Y);
  float* sBeta = reinterpret_cast<float*>(smem + L::BETA);
  float* sRed = reinterpret_cast<float*>(smem + L::RED);

  const E* qh = reinterpret_cast<const E*>(a.q) + (size_t)ci.t0 * rk + (size_t)h * DK;
  const E* kh = reinterpret_cast<const E*>(a.k) + (size_t)ci.t0 * rk + (size_t)h * DK;
  const E* lh = reinterpret_cast<const E*>(a.la) + (size_t)ci.t0 * rk + (size_t)h * DK;
  const E* bh = reinterpret_cast<const E*>(a.beta) + (size_t)ci.t0 * H + h;
  const float* gT = reinterpret_cast<const float*>(a.wsT) + blk * WB::TT;
  const float* gGm = a.wsG + blk * WB::G;
  const float* gA = a.wsdAqk + blk * WB::DAQK;
  const float* gTU = a.wsdTU + blk * WB::DTU;
  const float* gQS = a.wsdQS + blk * WB::DQS;
  const float* gKH = a.wsdKh + blk * WB::DKH;
  const float* gW = a.wsdW + blk * WB::DW;

  // ---- 1. loads: log_alpha -> g (cumsum), k, q rows; T, dAqk, dW; beta
  constexpr int NKS = DK / 32;
  const int r = 16 * w + r16;   // row held by this lane in the row-block layout
  float xk[NKS][8], xq[NKS][8], xl[NKS][8];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    load8<E>(kh + r * rk + 32 * ks + 8 * q4, r < len, xk[ks]);
    load8<E>(qh + r * rk + 32 * ks + 8 * q4, r < len, xq[ks]);
    load8<E>(lh + r * rk + 32 * ks + 8 * q4, r < len, xl[ks]);
  }
  if (tid < CH) sBeta[tid] = tid < len ? f32(bh[(size_t)tid * H]) : 0.f;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int c0 = 32 * ks + 8 * q4;
    *reinterpret_cast<f32x4*>(sG + r * L::LDG + c0) = f32x4{xl[ks][0], xl[ks][1], xl[ks][2], xl[ks][3]};
    *reinterpret_cast<f32x4*>(sG + r * L::LDG + c0 + 4) = f32x4{xl[ks][4], xl[ks][5], xl[ks][6], xl[ks][7]};
    store4<E>(sK + r * L::LDK + c0, xk[ks][0], xk[ks][1], xk[ks][2], xk[ks][3]);
    store4<E>(sK + r * L::LDK + c0 + 4, xk[ks][4], xk[ks][5], xk[ks][6], xk[ks][7]);
    store4<E>(sQ + r * L::LDK + c0, xq[ks][0], xq[ks][1], xq[ks][2], xq[ks][3]);
    store4<E>(sQ + r * L::LDK + c0 + 4, xq[ks][4], xq[ks][5], xq[ks][6], xq[ks][7]);
  }
  for (int o = tid; o < CH * CH; o += NT) {
    const int rr = o / CH, cc = o % CH;
    sT[rr * L::LDT + cc] = cvt<OP>(gT[o]);
    sA1[rr * L::LDA + cc] = gA[o];
  }
  for (int o = tid; o < CH * DK; o += NT) sDW[(o / DK) * L::LDO + o % DK] = cvt<OP>(gW[o]);
  __syncthreads();
  {
    constexpr int NSPLIT = NT / DK, RPS = CH / NSPLIT;
    const int c = tid % DK, s = tid / DK;
    float acc = 0.f;
    for (int rr = s * RPS; rr < (s + 1) * RPS; ++rr) {
      acc += sG[rr * L::LDG + c];
      sG[rr * L::LDG + c] = acc;
    }
    sRed[s * DK + c] = acc;
  }
  __syncthreads();
  {
    constexpr int NSPLIT = NT / DK, RPS = CH / NSPLIT;
    const int c = tid % DK, s = tid / DK;
    if (s > 0) {
      float off = 0.f;
      for (int s2 = 0; s2 < s; ++s2) off += sRed[s2 * DK + c];
      for (int rr = s * RPS; rr < (s + 1) * RPS; ++rr) sG[rr * L::LDG + c] += off;
    }
  }
  __syncthreads();
  // K+ = k * exp(g) (operand copy)
  for (int o = tid; o < CH * DK; o += NT) {
    const int rr = o / DK, cc = o % DK;
    sKp[rr * L::LDO + cc] = cvt<OP>(f32(sK[rr * L::LDK + cc]) * __expf(sG[rr * L::LDG + cc]));
  }
  __syncthreads();

  // per-lane C-tile layout: rows 16w + 4q4 + ii, columns 16nt + r16
  // ---- 2. T^T dW (token tile w, all channel tiles), and rowsum(K+ * T^T dW)
  f32x4 tdw[NKT];
  float dbeta[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nt = 0; nt < NKT; ++nt) {
    f32x4 x = zero4();
#pragma unroll
    for (int k = 0; k < CH; k += 32)
      x = mma(frag_col<OP>(sT, L::LDT, 16 * w + r16, k + 8 * q4), frag_col<OP>(sDW, L::LDO, 16 * nt + r16, k + 8 * q4), x);
    tdw[nt] = x;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int rr = 16 * w + 4 * q4 + ii, cc = 16 * nt + r16;
      dbeta[ii] += f32(sK[rr * L::LDK + cc]) * __expf(sG[rr * L::LDG + cc]) * x[ii];
    }
  }
  // ---- 3. dT = dW (b K+)^T + dT_U  (token tile w, 4 column tiles) -> sA2
  {
    f32x4 x[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      x[nt] = zero4();
#pragma unroll
      for (int k = 0; k < DK; k += 32)
        x[nt] = mma(frag_row<OP>(sDW, L::LDO, 16 * w + r16, k + 8 * q4), frag_row<OP>(sKp, L::LDO, 16 * nt + r16, k + 8 * q4),
                    x[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int rr = 16 * w + 4 * q4 + ii, cc = 16 * nt + r16;
        sA2[rr * L::LDA + cc] = x[nt][ii] * sBeta[cc] + gTU[rr * CH + cc];
      }
  }
  __syncthreads();  // dT complete; dW and K+ are dead
  // ---- 4. Y = dT T^T -> sY ; dA = -strict(T^T Y) ; dG = b dA -> sA2 ; rowsum(dA * G)
  {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4 x = zero4();
#pragma unroll
      for (int k = 0; k < CH; k += 32) {
        float y8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) y8[u] = sA2[(16 * w + r16) * L::LDA + k + 8 * q4 + u];
        x = mma(frag_from<OP>(y8), frag_row<OP>(sT, L::LDT, 16 * nt + r16, k + 8 * q4), x);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) sY[(16 * w + 4 * q4 + ii) * L::LDT + 16 * nt + r16] = cvt<OP>(x[ii]);
    }
  }
  __syncthreads();
  {
    f32x4 x[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      x[nt] = zero4();
#pragma unroll
      for (int k = 0; k < CH; k += 32)
        x[nt] = mma(frag_col<OP>(sT, L::LDT, 16 * w + r16, k + 8 * q4), frag_col<OP>(sY, L::LDT, 16 * nt + r16, k + 8 * q4),
                    x[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int rr = 16 * w + 4 * q4 + ii, cc = 16 * nt + r16;
        const float da = cc < rr ? -x[nt][ii] : 0.f;
        dbeta[ii] += da * gGm[rr * CH + cc];
        sA2[rr * L::LDA + cc] = sBeta[rr] * da;   // dG (each element written by its only reader-to-be later)
      }
  }
  __syncthreads();

  // ---- 5. gated products with per-block reference rows (split bf16 operands)
  // row side, block a = w: dq_g = e^{g_r - g_m} (dAqk . R_a), dkp_g = e^{g_r - g_m} (dG . R_a),
  // R_a[i] = k_i e^{g_m - g_i}; column side, block b = w:
  // dkm = sum_{a >= b} e^{g_m(a) - g_i} ((dAqk_a^T q_a + dG_a^T k_a) e^{g_a - g_m(a)})
  f32x4 dqg[NKT], dkpg[NKT], dkm[NKT];
#pragma unroll
  for (int nt = 0; nt < NKT; ++nt) dqg[nt] = dkpg[nt] = dkm[nt] = zero4();
  {
    const int ab = w, ref = 16 * ab + 8;
    const int kmax = 16 * (ab + 1);  // columns i < kmax can be nonzero
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) {
      const int cc = 16 * nt + r16;
      for (int k = 0; k < kmax; k += 32) {
        const SFrag<SE> fa1 = sfrag_row<SE>(sA1, L::LDA, 16 * ab + r16, k + 8 * q4);
        const SFrag<SE> fa2 = sfrag_row<SE>(sA2, L::LDA, 16 * ab + r16, k + 8 * q4);
        float xr[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = k + 8 * q4 + u;
          xr[u] = i < kmax ? f32(sK[i * L::LDK + cc]) * __expf(sG[ref * L::LDG + cc] - sG[i * L::LDG + cc]) : 0.f;
        }
        const SFrag<SE> fr = sfrag_from<SE>(xr);
        dqg[nt] = mma_ss(fa1, fr, dqg[nt]);
        dkpg[nt] = mma_ss(fa2, fr, dkpg[nt]);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int rr = 16 * ab + 4 * q4 + ii;
        const float e = __expf(sG[rr * L::LDG + cc] - sG[ref * L::LDG + cc]);
        dqg[nt][ii] *= e;
        dkpg[nt][ii] *= e;
      }
    }
  }
  {
    const int b = w;
    for (int ab = b; ab < 4; ++ab) {
      const int ref = 16 * ab + 8;
#pragma unroll
      for (int nt = 0; nt < NKT; ++nt) {
        const int cc = 16 * nt + r16;
        // A[m = i][k = r'] : r' < 16 -> dAqk[16a + r'][i], r' >= 16 -> dG[16a + r' - 16][i]
        const float* srcA = q4 < 2 ? sA1 : sA2;
        const int rbase = 16 * ab + 8 * (q4 & 1);
        const SFrag<SE> fa = sfrag_col_f32<SE>(srcA, L::LDA, 16 * b + r16, rbase);
        float xl8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int rr = rbase + u;
          const float src = q4 < 2 ? f32(sQ[rr * L::LDK + cc]) : f32(sK[rr * L::LDK + cc]);
          xl8[u] = src * __expf(sG[rr * L::LDG + cc] - sG[ref * L::LDG + cc]);
        }
        const f32x4 y = mma_ss(fa, sfrag_from<SE>(xl8), zero4());
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int i = 16 * b + 4 * q4 + ii;
          dkm[nt][ii] += __expf(sG[ref * L::LDG + cc] - sG[i * L::LDG + cc]) * y[ii];
        }
      }
    }
  }

  // ---- 6. assembly: dq, dk, dg (rows 16w + 4q4 + ii, channel tiles nt)
  O* dqh = reinterpret_cast<O*>(a.dq) + (size_t)ci.t0 * rk + (size_t)h * DK;
  O* dkh_ = reinterpret_cast<O*>(a.dk_) + (size_t)ci.t0 * rk + (size_t)h * DK;
  O* dlh = reinterpret_cast<O*>(a.dla) + (size_t)ci.t0 * rk + (size_t)h * DK;
  float dgv[NKT][4];
  float khs[NKT];   // column sums over this lane's rows of dKh * Kh  (for dg_C)
#pragma unroll
  for (int nt = 0; nt < NKT; ++nt) {
    khs[nt] = 0.f;
    const int cc = 16 * nt + r16;
    const float gl = sG[(CH - 1) * L::LDG + cc];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int rr = 16 * w + 4 * q4 + ii;
      const float g = sG[rr * L::LDG + cc];
      const float eg = __expf(g);
      const float kv = f32(sK[rr * L::LDK + cc]), qv = f32(sQ[rr * L::LDK + cc]);
      const float dq = eg * gQS[rr * DK + cc] + dqg[nt][ii];
      const float dkp = eg * sBeta[rr] * tdw[nt][ii] + dkpg[nt][ii];
      const float dkmv = dkm[nt][ii];
      const float dkh = __expf(gl - g) * gKH[rr * DK + cc];
      const float dk = dkp + dkmv + dkh;
      dgv[nt][ii] = dq * qv + (dkp - dkmv - dkh) * kv;
      khs[nt] += dkh * kv;
      if (rr < len) {
        dqh[(size_t)rr * rk + cc] = cvt<O>(dq);
        dkh_[(size_t)rr * rk + cc] = cvt<O>(dk);
      }
    }
  }
  // rowsums for dbeta: reduce over the 16 column lanes, then over nothing else
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    float p = dbeta[ii];
    p += __shfl_xor(p, 1);
    p += __shfl_xor(p, 2);
    p += __shfl_xor(p, 4);
    p += __shfl_xor(p, 8);
    dbeta[ii] = p;
  }
  __syncthreads();  // all reads of g done before dg overwrites it
  // dg -> LDS (sG region), column sums of dKh*Kh -> sRed
#pragma unroll
  for (int nt = 0; nt < NKT; ++nt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) sG[(16 * w + 4 * q4 + ii) * L::LDG + 16 * nt + r16] = dgv[nt][ii];
  {
    // reduce khs over q4 (lanes differing in bits 4,5) then over waves via sRed
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) {
      float p = khs[nt];
      p += __shfl_xor(p, 16);
      p += __shfl_xor(p, 32);
      if (q4 == 0) sRed[w * DK + 16 * nt + r16] = p;
    }
  }
  if (r16 == 0) {
    const float* gbv = a.wsdBv + blk * WB::DBV;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int rr = 16 * w + 4 * q4 + ii;
      if (rr < len) reinterpret_cast<O*>(a.dbeta)[((size_t)ci.t0 + rr) * H + h] = cvt<O>(dbeta[ii] + gbv[rr]);
    }
  }
  __syncthreads();
  // dg_C terms on the last row, then the reverse cumulative sum over rows -> dlog_alpha
  if (tid < DK) {
    const int c = tid;
    float s = 0.f;
    for (int ww = 0; ww < 4; ++ww) s += sRed[ww * DK + c];
    const float gl_exp = a.wsGam[blk * WB::GAM + c];
    sG[(CH - 1) * L::LDG + c] += s + a.wsdGam[blk * WB::DGAM + c] * gl_exp;
  }
  __syncthreads();
  {
    constexpr int NSPLIT = NT / DK, RPS = CH / NSPLIT;
    const int c = tid % DK, s = tid / DK;
    float acc = 0.f;
    for (int rr = (s + 1) * RPS - 1; rr >= s * RPS; --rr) acc += sG[rr * L::LDG + c];
    sRed[s * DK + c] = acc;   // total of this part
  }
  __syncthreads();
  {
    constexpr int NSPLIT = NT / DK, RPS = CH / NSPLIT;
    const int c = tid % DK, s = tid / DK;
    float acc = 0.f;
    for (int s2 = s + 1; s2 < NSPLIT; ++s2) acc += sRed[s2 * DK + c];
    for (int rr = (s + 1) * RPS - 1; rr >= s * RPS; --rr) {
      acc += sG[rr * L::LDG + c];
      if (rr < len) dlh[(size_t)rr * rk + c] = cvt<O>(acc);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename E, typename O, int DK, int DV>
hipError_t launch_bwd(const Args& a, hipStream_t st) {
  hipError_t e = launch_bwd_front<E, DK, DV>(a, st);
  if (e != hipSuccess) return e;
  constexpr int DVS = 16, NSL = DV / DVS;
  const int units = a.N * a.H;
  const int grid = (units + 7) / 8 * 8 * NSL;
  if (grid > 0) {
    KDA_TIMED("kda_state_bwd_revpass", st,
              hipLaunchKernelGGL((kda_state_rev<E, DK, DV, DVS>), dim3(grid), dim3(512), 0, st, a));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.max_chunks > 0) {
    KDA_TIMED("kda_bwd_dv", st, hipLaunchKernelGGL((kda_bwd_dv<E, O, DK, DV>), dim3(a.max_chunks, a.H), dim3(256), 0, st, a));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    KDA_TIMED("kda_bwd_dk", st, hipLaunchKernelGGL((kda_bwd_dk<E, O, DK, DV>), dim3(a.max_chunks, a.H), dim3(256), 0, st, a));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

#define KDA_INST(E, O, DK, DV) template hipError_t launch_bwd<E, O, DK, DV>(const Args&, hipStream_t);
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
