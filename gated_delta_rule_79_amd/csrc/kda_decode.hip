// kda_decode.hip -- decode / replay step of the KDA recurrence on gfx950.
//
// fireworks.ai, "Kimi K3 on Fireworks: Fast RL at frontier scale": the section
// on Kimi Delta Attention gives KDA a fixed-size decoding state, and the
// section on speculative decoding keeps that state consistent after rejected
// draft tokens by replaying the state-update inputs of the accepted tokens
// from a committed state rather than snapshotting the state per candidate.
//
// One call advances B sequences by T (<= KDA_DECODE_MAX_TOKENS) tokens each,
// token by token, from states held in a caller-owned pool:
//     P = Diag(exp(log_alpha_t)) S,  delta = v_t - P^T k_t,
//     S = P + beta_t k_t delta^T,    o_t = scale S^T q_t,
// writes every o_t, and stores the state after the first num_commit[b] tokens
// back into the sequence's pool slot.  A verification pass commits nothing;
// the replay after acceptance commits the accepted prefix.
//
// Work split: one 256-thread work-group per (sequence, head).  The fp32 state
// stays in registers for all T tokens: thread (rg, cg) holds columns 4cg..4cg+3
// of rows rg, rg + RG, ...; a wave's float4 loads cover whole rows, so the
// state moves through HBM once each way in 1 KB contiguous pieces.  The two
// contractions over the key channel (P^T k and P^T q) are reduced together:
// across the row groups of a wave with lane shuffles, then across the eight
// waves through LDS, in a fixed order (bitwise reproducible).  S^T q needs no
// second reduction: S^T q = P^T q + beta delta (k . q).
#include "kda.h"
#include "kda_internal.hpp"

namespace kda {

namespace {

#ifndef KDA_DECODE_NT
#define KDA_DECODE_NT 256   // threads per (sequence, head) work-group (512: 0.246 ms against 0.237 ms
                            // for 512 sequences x 4 tokens; 1,024: 0.389 ms)
#endif
constexpr int DEC_NT = KDA_DECODE_NT;
constexpr int DEC_NW = DEC_NT / 64;

__device__ __forceinline__ float4 shfl_xor4(float4 x, int m) {
  return make_float4(__shfl_xor(x.x, m), __shfl_xor(x.y, m), __shfl_xor(x.z, m), __shfl_xor(x.w, m));
}

template <typename O> __device__ __forceinline__ void store4(O* p, float4 x);
template <> __device__ __forceinline__ void store4<float>(float* p, float4 x) {
  *reinterpret_cast<float4*>(p) = x;
}
template <> __device__ __forceinline__ void store4<bf16>(bf16* p, float4 x) {
  bf16x4 y;
  y[0] = cvt<bf16>(x.x);
  y[1] = cvt<bf16>(x.y);
  y[2] = cvt<bf16>(x.z);
  y[3] = cvt<bf16>(x.w);
  *reinterpret_cast<bf16x4*>(p) = y;
}

}  // namespace

// MT: token capacity of the LDS staging (4 for the usual 1..4-token steps, so
// more work-groups fit on a CU; KDA_DECODE_MAX_TOKENS otherwise).
template <typename E, typename O, int DK, int DV, int MT>
__global__ __launch_bounds__(DEC_NT) void kda_decode_step(const DecodeArgs a) {
  constexpr int CG = DV / 4;          // float4 column groups
  constexpr int RG = DEC_NT / CG;     // row groups (8 or 16 with 256 threads)
  constexpr int NR = DK / RG;         // state rows per thread
  static_assert(DK % RG == 0 && 64 % CG == 0, "decode thread layout");
  __shared__ float sQ[MT][DK], sK[MT][DK], sA[MT][DK], sV[MT][DV];
  __shared__ float sB[MT], sQK[MT];
  __shared__ float4 sRed[2][DEC_NW][2][CG];   // [token parity][wave][P^T k | P^T q][column group]

  const int H = a.H, T = a.T;
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG, w = wave_id(), lane = lane_id();
  const int slot = a.idx ? a.idx[b] : b;
  O* out = reinterpret_cast<O*>(a.out);
  if (slot < 0 || slot >= a.pool_size) {   // padding entry: zero outputs, no state touched
    for (int o = tid; o < T * DV; o += DEC_NT) {
      const int t = o / DV, j = o % DV;
      out[((size_t)(b * T + t) * H + h) * DV + j] = cvt<O>(0.f);
    }
    return;
  }
  int ncommit = a.ncommit ? a.ncommit[b] : T;
  ncommit = ncommit < 0 ? 0 : (ncommit > T ? T : ncommit);

  // state slice of this thread: rows rg + i * RG, columns 4cg .. 4cg + 3
  float* Sg = a.pool + ((size_t)slot * H + h) * DK * DV + 4 * cg;
  float4 S[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {   // streamed once: non-temporal, so it does not displace reused lines
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sg + (size_t)(rg + i * RG) * DV));
    S[i] = make_float4(x[0], x[1], x[2], x[3]);
  }

  // the tokens' vectors, in fp32 (decays already exponentiated)
  const E* q = reinterpret_cast<const E*>(a.q);
  const E* k = reinterpret_cast<const E*>(a.k);
  const E* la = reinterpret_cast<const E*>(a.la);
  const E* v = reinterpret_cast<const E*>(a.v);
  for (int o = tid; o < T * DK; o += DEC_NT) {
    const int t = o / DK, c = o % DK;
    const size_t g = ((size_t)(b * T + t) * H + h) * DK + c;
    sQ[t][c] = f32(q[g]);
    sK[t][c] = f32(k[g]);
    const float x = f32(la[g]);
    const float al = a.gate_ls ? 1.f / (1.f + __expf(-x)) : __expf(x);   // alpha = sigmoid(x) for a raw gate
    sA[t][c] = al < ALPHA_FLOOR ? ALPHA_FLOOR : al;   // the floor of log alpha the chunked kernels apply
  }
  for (int o = tid; o < T * DV; o += DEC_NT) {
    const int t = o / DV, j = o % DV;
    sV[t][j] = f32(v[((size_t)(b * T + t) * H + h) * DV + j]);
  }
  if (tid < T) sB[tid] = f32(reinterpret_cast<const E*>(a.beta)[(size_t)(b * T + tid) * H + h]);
  __syncthreads();
  if (a.qk_norm) {   // q, k rows to unit L2 norm (fp32), one wave per row
    for (int row = w; row < 2 * T; row += DEC_NW) {
      float* x = row < T ? sQ[row] : sK[row - T];
      float ss = 0.f;
      for (int c = lane; c < DK; c += 64) ss += x[c] * x[c];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
      const float sc = 1.0f / sqrtf(ss + L2N_EPS);
      for (int c = lane; c < DK; c += 64) x[c] *= sc;
    }
    __syncthreads();
  }
  for (int t = w; t < T; t += DEC_NW) {   // k_t . q_t, one wave per token
    float p = 0.f;
    for (int c = lane; c < DK; c += 64) p += sQ[t][c] * sK[t][c];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) p += __shfl_xor(p, m);
    if (lane == 0) sQK[t] = p;
  }
  __syncthreads();

  const float scale = a.scale;
  for (int t = 0; t < T; ++t) {
    float4 kp = make_float4(0.f, 0.f, 0.f, 0.f), qp = kp;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int r = rg + i * RG;
      const float al = sA[t][r], kr = sK[t][r], qr = sQ[t][r];
      S[i].x *= al;
      S[i].y *= al;
      S[i].z *= al;
      S[i].w *= al;
      kp.x += kr * S[i].x;
      kp.y += kr * S[i].y;
      kp.z += kr * S[i].z;
      kp.w += kr * S[i].w;
      qp.x += qr * S[i].x;
      qp.y += qr * S[i].y;
      qp.z += qr * S[i].z;
      qp.w += qr * S[i].w;
    }
#pragma unroll
    for (int m = CG; m < 64; m <<= 1) {   // row groups sharing a wave
      const float4 x = shfl_xor4(kp, m), y = shfl_xor4(qp, m);
      kp.x += x.x; kp.y += x.y; kp.z += x.z; kp.w += x.w;
      qp.x += y.x; qp.y += y.y; qp.z += y.z; qp.w += y.w;
    }
    const int buf = t & 1;   // alternate buffers: one barrier per token suffices
    if (lane < CG) {
      sRed[buf][w][0][cg] = kp;
      sRed[buf][w][1][cg] = qp;
    }
    __syncthreads();
    float4 pk = sRed[buf][0][0][cg], pq = sRed[buf][0][1][cg];
#pragma unroll
    for (int ww = 1; ww < DEC_NW; ++ww) {
      const float4 x = sRed[buf][ww][0][cg], y = sRed[buf][ww][1][cg];
      pk.x += x.x; pk.y += x.y; pk.z += x.z; pk.w += x.w;
      pq.x += y.x; pq.y += y.y; pq.z += y.z; pq.w += y.w;
    }
    const float bt = sB[t], bqk = bt * sQK[t];
    const float4 vv = *reinterpret_cast<const float4*>(&sV[t][4 * cg]);
    const float4 dl = make_float4(vv.x - pk.x, vv.y - pk.y, vv.z - pk.z, vv.w - pk.w);
    if (rg == 0) {
      const float4 o = make_float4(scale * (pq.x + bqk * dl.x), scale * (pq.y + bqk * dl.y),
                                   scale * (pq.z + bqk * dl.z), scale * (pq.w + bqk * dl.w));
      store4<O>(out + ((size_t)(b * T + t) * H + h) * DV + 4 * cg, o);
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float bk = bt * sK[t][rg + i * RG];
      S[i].x += bk * dl.x;
      S[i].y += bk * dl.y;
      S[i].z += bk * dl.z;
      S[i].w += bk * dl.w;
    }
    if (t + 1 == ncommit) {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const f32x4 x = {S[i].x, S[i].y, S[i].z, S[i].w};
        __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(Sg + (size_t)(rg + i * RG) * DV));
      }
    }
  }
}

template <typename E, typename O, int DK, int DV>
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  const long long units = (long long)a.B * a.H;
  if (units == 0 || a.T == 0) return hipSuccess;
  if (a.T <= 4)
    KDA_TIMED("kda_decode_step", st,
              hipLaunchKernelGGL((kda_decode_step<E, O, DK, DV, 4>), dim3((unsigned)units), dim3(DEC_NT), 0, st, a));
  else
    KDA_TIMED("kda_decode_step", st,
              hipLaunchKernelGGL((kda_decode_step<E, O, DK, DV, KDA_DECODE_MAX_TOKENS>), dim3((unsigned)units),
                                 dim3(DEC_NT), 0, st, a));
  return hipGetLastError();
}

#define KDA_DECODE_INST(E, O, DK, DV) template hipError_t launch_decode<E, O, DK, DV>(const DecodeArgs&, hipStream_t);
#define KDA_DECODE_DIMS(E, O) \
  KDA_DECODE_INST(E, O, 64, 64) KDA_DECODE_INST(E, O, 64, 128) KDA_DECODE_INST(E, O, 128, 64) KDA_DECODE_INST(E, O, 128, 128)
KDA_DECODE_DIMS(float, float)
KDA_DECODE_DIMS(bf16, float)
KDA_DECODE_DIMS(bf16, bf16)
#undef KDA_DECODE_DIMS
#undef KDA_DECODE_INST

}  // namespace kda
