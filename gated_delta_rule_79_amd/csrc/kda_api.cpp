// kda_api.cpp -- C ABI of libkda.so: validation, workspace planning, dispatch.
//
// Everything here runs on the host before any launch; errors return a status
// and enqueue nothing.  See include/kda.h for the contract.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kda_internal.hpp"
#include "kda_conv.hpp"

namespace {

using kda::Args;
using kda::bf16;
using kda::CH;
using kda::ChunkInfo;

constexpr size_t ALIGN = 256;
constexpr int32_t KDA_PREP_FLAGS = KDA_FLAG_QK_L2NORM | KDA_FLAG_GATE_LOGSIGMOID;
size_t up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Plan {
  int N = 0;
  int max_chunks = 0;
  size_t esz = 0;
  size_t chunks = 0, sc0 = 0, so = 0, W = 0, KhT = 0, Qt = 0, Ut = 0, Aqk = 0, Gam = 0, steep = 0;
  size_t T = 0, UtF = 0, G = 0, KhF = 0, KhTL = 0, S = 0, U = 0, dS = 0, dU = 0, DQK = 0, GS = 0;
  int segs = 1;
  size_t vsc0 = 0, vord = 0, seg_in = 0, seg_loc = 0, seg_m = 0;
  size_t total = 0;
};

bool dims_ok(const kda_desc* d) {
  return (d->dk == 64 || d->dk == 128) && (d->dv == 64 || d->dv == 128) &&
         (d->dtype == KDA_F32 || d->dtype == KDA_BF16) &&
         (d->out_dtype == KDA_F32 || (d->out_dtype == KDA_BF16 && d->dtype == KDA_BF16));
}

// Number of sequences and chunk slots; varlen when `varlen`.  Sizes are taken in
// 64 bits and bounded so that every work-item count and launch grid derived from
// them (chunk slots x heads; sequences x heads x value slices x stretches, at most
// 64 stretches and 8 slices) fits an int.
bool shape_of(const kda_desc* d, bool varlen, int* N, int* max_chunks) {
  if (d->B < 1 || d->T < 0 || d->H < 1 || d->H > 65535) return false;
  const long long tok = (long long)d->B * d->T;
  if (tok >= (1LL << 31)) return false;
  long long n, mc;
  if (varlen) {
    if (d->B != 1 || d->num_seqs < 1) return false;
    n = d->num_seqs;
    mc = (long long)d->T / CH + n;
  } else {
    n = d->B;
    mc = (long long)d->B * (((long long)d->T + CH - 1) / CH);
  }
  if (mc * d->H >= (1LL << 31) || n * d->H >= (1LL << 22)) return false;
  *N = (int)n;
  *max_chunks = (int)mc;
  return true;
}

Plan make_plan(const kda_desc* d, bool bwd, int N, int max_chunks) {
  Plan p;
  p.N = N;
  p.max_chunks = max_chunks;
  p.esz = d->dtype == KDA_BF16 ? 2 : 4;
  const size_t nb = (size_t)max_chunks * d->H;  // chunk-head blocks
  const size_t dk = d->dk, dv = d->dv, e = p.esz;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += up(bytes); return at; };
  p.chunks = take((size_t)max_chunks * sizeof(ChunkInfo));
  p.sc0 = take((size_t)(N + 1) * sizeof(int32_t));
  p.so = take((size_t)N * sizeof(int32_t));
  p.W = take(nb * CH * dk * e);    // operand type: fp16 for bf16 inputs, fp32 otherwise
  p.KhT = take(nb * dk * CH * e);
  p.Qt = take(nb * CH * dk * e);
  p.Ut = take(nb * dv * CH * e);
  p.Aqk = take(nb * CH * CH * e);
  p.Gam = take(nb * dk * 4);
  p.steep = take(nb * 4);
  if (bwd) {
    p.T = take(nb * CH * CH * e);   // operand type
    p.UtF = take(nb * dv * CH * 4);
    p.G = take(nb * CH * CH * 4);
    p.KhF = take(nb * CH * dk * 4);
    if (e == 2) p.KhTL = take(nb * dk * CH * e);   // Kh^T lo half (split training-mode state update)
    p.S = take(nb * dk * dv * 4);
    p.U = take(nb * dv * CH * 4);
    p.dS = take(nb * dk * dv * 4);
    p.dU = take(nb * dv * CH * 4);
    if (d->flags & KDA_FLAG_QK_L2NORM) p.DQK = take(nb * 2 * CH * dk * 4);   // dq^, dk^ before the norm's chain rule
    p.GS = take((2 + kda::GS_PARTS) * 4);   // gradient scale (s, 1/s) and the pre-pass's partial maxima
  }
  // segment scan buffers (the same stretches for a training-mode forward and the
  // backward, which reuses the forward's transfers)
  p.segs = kda::fwd_segments(N, d->H, d->dv, (long long)d->B * d->T, bwd);
  if (p.segs > 1) {
    const size_t nv = (size_t)N * p.segs;
    p.vsc0 = take((nv + 1) * sizeof(int32_t));
    p.vord = take(nv * sizeof(int32_t));
    p.seg_in = take(nv * d->H * dk * dv * 4);
    p.seg_loc = take(nv * d->H * dk * dv * 4);
    p.seg_m = take(nv * d->H * dk * dk * 4);
  }
  p.total = o;
  return p;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  return s && *s ? std::atoi(s) : dflt;
}

// Optional synchronous check of cu_seqlens contents (KDA_DEBUG=1).
bool cu_ok(const int32_t* cu, int N, int T, hipStream_t st) {
  std::vector<int32_t> h((size_t)N + 1);
  if (hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess) return false;
  if (hipStreamSynchronize(st) != hipSuccess) return false;
  if (h[0] != 0 || h[N] != T) return false;
  for (int i = 0; i < N; ++i)
    if (h[i + 1] < h[i]) return false;
  return true;
}

void fill_ws(Args& a, const Plan& p, void* ws) {
  char* b = static_cast<char*>(ws);
  a.chunks = reinterpret_cast<ChunkInfo*>(b + p.chunks);
  a.seq_chunk0 = reinterpret_cast<int32_t*>(b + p.sc0);
  a.seq_order = reinterpret_cast<int32_t*>(b + p.so);
  a.wsW = b + p.W;
  a.wsKhT = b + p.KhT;
  a.wsQt = b + p.Qt;
  a.wsUt = b + p.Ut;
  a.wsAqk = b + p.Aqk;
  a.wsGam = reinterpret_cast<float*>(b + p.Gam);
  a.steep = reinterpret_cast<int32_t*>(b + p.steep);
  auto fptr = [&](size_t off) { return off ? reinterpret_cast<float*>(b + off) : nullptr; };
  a.wsT = p.T ? b + p.T : nullptr;
  a.wsUtF = fptr(p.UtF);
  a.wsG = fptr(p.G);
  a.wsKhF = fptr(p.KhF);
  a.wsKhTL = p.KhTL ? b + p.KhTL : nullptr;
  a.wsS = fptr(p.S);
  a.wsU = fptr(p.U);
  a.wsdS = fptr(p.dS);
  a.wsdU = fptr(p.dU);
  a.wsDQK = fptr(p.DQK);
  if (p.GS && p.esz == 2) {   // the fp32 backward narrows nothing: no scale
    a.gscale = fptr(p.GS);
    a.gs_part = a.gscale + 2;
  }
  a.segs = p.segs;
  a.vsc0 = p.vsc0 ? reinterpret_cast<int32_t*>(b + p.vsc0) : nullptr;
  a.vord = p.vord ? reinterpret_cast<int32_t*>(b + p.vord) : nullptr;
  a.seg_in = fptr(p.seg_in);
  a.seg_loc = fptr(p.seg_loc);
  a.seg_m = fptr(p.seg_m);
}

hipError_t run_fwd(const kda_desc* d, const Args& a, hipStream_t st) {
  const bool bf = d->dtype == KDA_BF16, obf = d->out_dtype == KDA_BF16;
  const bool save = (d->flags & KDA_FLAG_SAVE_FOR_BACKWARD) != 0;
#define KDA_CASE(DK, DV)                                                                        \
  if (d->dk == DK && d->dv == DV)                                                               \
    return bf ? (obf ? kda::launch_fwd<bf16, bf16, DK, DV>(a, st, save)                         \
                     : kda::launch_fwd<bf16, float, DK, DV>(a, st, save))                       \
              : kda::launch_fwd<float, float, DK, DV>(a, st, save);
  KDA_CASE(64, 64)
  KDA_CASE(64, 128)
  KDA_CASE(128, 64)
  KDA_CASE(128, 128)
#undef KDA_CASE
  return hipErrorInvalidValue;
}

hipError_t run_bwd(const kda_desc* d, const Args& a, hipStream_t st) {
  const bool bf = d->dtype == KDA_BF16, obf = d->out_dtype == KDA_BF16;
  const bool saved = (d->flags & KDA_FLAG_USE_SAVED) != 0;
  if (bf) {
#define KDA_CASE(DK, DV)                                                                        \
    if (d->dk == DK && d->dv == DV)                                                             \
      return obf ? kda::launch_bwd<bf16, bf16, DK, DV>(a, st, saved)                            \
                 : kda::launch_bwd<bf16, float, DK, DV>(a, st, saved);
    KDA_CASE(64, 64)
    KDA_CASE(64, 128)
    KDA_CASE(128, 64)
    KDA_CASE(128, 128)
#undef KDA_CASE
  } else {  // fp32 backward is built for dk = 64 (the host check rejects dk = 128)
    if (d->dk == 64 && d->dv == 64) return kda::launch_bwd<float, float, 64, 64>(a, st, saved);
    if (d->dk == 64 && d->dv == 128) return kda::launch_bwd<float, float, 64, 128>(a, st, saved);
  }
  return hipErrorInvalidValue;
}

hipError_t run_decode(const kda_desc* d, const kda::DecodeArgs& a, hipStream_t st) {
  const bool bf = d->dtype == KDA_BF16, obf = d->out_dtype == KDA_BF16;
#define KDA_CASE(DK, DV)                                                                        \
  if (d->dk == DK && d->dv == DV)                                                               \
    return bf ? (obf ? kda::launch_decode<bf16, bf16, DK, DV>(a, st)                            \
                     : kda::launch_decode<bf16, float, DK, DV>(a, st))                          \
              : kda::launch_decode<float, float, DK, DV>(a, st);
  KDA_CASE(64, 64)
  KDA_CASE(64, 128)
  KDA_CASE(128, 64)
  KDA_CASE(128, 128)
#undef KDA_CASE
  return hipErrorInvalidValue;
}

// Short convolution: checks shared by the three entry points.
bool conv_desc_ok(const kda_conv_desc* d) {
  return d->W >= 2 && d->W <= 4 && d->D > 0 && d->D % 8 == 0 &&
         (d->dtype == KDA_F32 || d->dtype == KDA_BF16) &&
         (d->out_dtype == KDA_F32 || (d->out_dtype == KDA_BF16 && d->dtype == KDA_BF16)) &&
         (d->activation == KDA_CONV_IDENTITY || d->activation == KDA_CONV_SILU);
}

// Sequences of a forward/backward call; false on a bad shape.
bool conv_shape(const kda_conv_desc* d, bool varlen, int* N) {
  if (d->B < 1 || d->T < 0) return false;
  if ((long long)d->B * d->T * d->D >= (1LL << 40) || (long long)d->B * d->T >= (1LL << 31)) return false;
  if (varlen) {
    if (d->B != 1 || d->num_seqs < 1) return false;
    *N = d->num_seqs;
  } else {
    *N = d->B;
  }
  return *N <= 65535;
}

size_t conv_ws_bytes(const kda_conv_desc* d) {
  const long long tok = (long long)d->B * d->T;
  const size_t tiles = (size_t)((tok + kda::CONV_BWD_TILE - 1) / kda::CONV_BWD_TILE);
  return tiles * (size_t)(d->W + 1) * (size_t)d->D * sizeof(float);
}

void conv_args(kda::ConvArgs& c, const kda_conv_desc* d, int N) {
  std::memset(&c, 0, sizeof c);
  c.B = d->B;
  c.T = d->T;
  c.D = d->D;
  c.N = N;
  c.tokens = d->B * d->T;
  c.silu = d->activation == KDA_CONV_SILU;
}

enum class ConvOp { Fwd, Bwd, Decode };
hipError_t run_conv(const kda_conv_desc* d, const kda::ConvArgs& c, ConvOp op, hipStream_t st) {
  const bool bf = d->dtype == KDA_BF16, obf = d->out_dtype == KDA_BF16;
#define KDA_CONV_CALL(E, O, W)                                                   \
  return op == ConvOp::Fwd   ? kda::launch_conv_fwd<E, O, W>(c, st)              \
         : op == ConvOp::Bwd ? kda::launch_conv_bwd<E, O, W>(c, st)              \
                             : kda::launch_conv_decode<E, O, W>(c, st);
#define KDA_CONV_CASE(KW)                                \
  if (d->W == KW) {                                      \
    if (!bf) { KDA_CONV_CALL(float, float, KW) }         \
    if (obf) { KDA_CONV_CALL(bf16, bf16, KW) }           \
    KDA_CONV_CALL(bf16, float, KW)                       \
  }
  KDA_CONV_CASE(2)
  KDA_CONV_CASE(3)
  KDA_CONV_CASE(4)
#undef KDA_CONV_CASE
#undef KDA_CONV_CALL
  return hipErrorInvalidValue;
}

void base_args(Args& a, const kda_desc* d, int N, int max_chunks) {
  std::memset(&a, 0, sizeof a);
  a.qk_norm = (d->flags & KDA_FLAG_QK_L2NORM) != 0;
  a.gate_ls = (d->flags & KDA_FLAG_GATE_LOGSIGMOID) != 0;
  a.B = d->B;
  a.T = d->T;
  a.H = d->H;
  a.dk = d->dk;
  a.dv = d->dv;
  a.N = N;
  a.max_chunks = max_chunks;
  a.scale = d->scale != 0.f ? d->scale : 1.0f / std::sqrt((float)d->dk);
  a.dvs = 16;
  a.out_bf16 = d->out_dtype == KDA_BF16;
}

// ---- opt-in per-kernel timing -------------------------------------------
struct TimingState {
  std::mutex mu;
  bool on = false;
  struct Pending { const char* name; hipEvent_t a, b; };
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  std::map<std::string, std::pair<double, int>> totals;
  std::vector<const char*> order;  // static kernel-name literals, first-seen order
  const char* open_name = nullptr;
  hipEvent_t open_ev = nullptr;
  bool failed = false;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) failed = true;
    return e;
  }
};
TimingState& timing() {
  static TimingState t;
  return t;
}

// First failing launch of the current kda_fwd/kda_bwd call on this host thread.
thread_local char tl_error[256];
void clear_error() { tl_error[0] = 0; }
kda_status launch_status(hipError_t e) {
  if (e == hipSuccess) return KDA_SUCCESS;
  if (!tl_error[0]) std::snprintf(tl_error, sizeof tl_error, "%s (%s)", hipGetErrorName(e), hipGetErrorString(e));
  return KDA_ERROR_LAUNCH;
}

}  // namespace

namespace kda {
void note_launch(const char* name) {
  const hipError_t e = hipPeekAtLastError();
  if (e == hipSuccess || tl_error[0]) return;
  std::snprintf(tl_error, sizeof tl_error, "%s: %s (%s)", name, hipGetErrorName(e), hipGetErrorString(e));
}
void timing_begin(const char* name, hipStream_t st) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.on) return;
  t.open_name = name;
  t.open_ev = t.get();
  if (t.open_ev && hipEventRecord(t.open_ev, st) != hipSuccess) t.failed = true;
}
void timing_end(hipStream_t st) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.on || !t.open_ev) return;
  hipEvent_t b = t.get();
  if (b && hipEventRecord(b, st) != hipSuccess) t.failed = true;
  t.pending.push_back({t.open_name, t.open_ev, b});
  t.open_ev = nullptr;
}
}  // namespace kda

extern "C" {

void kda_timing_enable(int enable) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.on = enable != 0;
  if (t.on) {
    for (auto& p : t.pending) {
      t.pool.push_back(p.a);
      t.pool.push_back(p.b);
    }
    t.pending.clear();
    t.totals.clear();
    t.order.clear();
    t.failed = false;
  }
}

int kda_timing_read(int max_entries, const char** names, double* total_ms, int* launches) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  for (auto& p : t.pending) {
    float ms = 0.f;
    if (!p.a || !p.b || hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess)
      t.failed = true;
    auto it = t.totals.find(p.name);
    if (it == t.totals.end()) {
      t.order.push_back(p.name);
      it = t.totals.emplace(p.name, std::make_pair(0.0, 0)).first;
    }
    it->second.first += ms;
    it->second.second += 1;
    t.pool.push_back(p.a);
    t.pool.push_back(p.b);
  }
  t.pending.clear();
  if (t.failed) return -1;
  int n = 0;
  for (const char* nm : t.order) {
    if (n >= max_entries) break;
    const auto& v = t.totals[nm];
    if (names) names[n] = nm;
    if (total_ms) total_ms[n] = v.first;
    if (launches) launches[n] = v.second;
    ++n;
  }
  return n;
}


const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_SUCCESS: return "success";
    case KDA_ERROR_INVALID_VALUE: return "invalid value";
    case KDA_ERROR_NOT_SUPPORTED: return "not supported (dk, dv must be 64 or 128; dtype f32 or bf16; bf16 out_dtype needs bf16 inputs)";
    case KDA_ERROR_MISALIGNED: return "pointer not 16-byte aligned";
    case KDA_ERROR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KDA_ERROR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* kda_last_error(void) { return tl_error; }

size_t kda_workspace_bytes(const kda_desc* d, int backward) {
  if (!d || !dims_ok(d)) return 0;
  int N, mc;
  size_t best = 0;
  if (shape_of(d, false, &N, &mc)) best = make_plan(d, backward != 0, N, mc).total;
  if (d->num_seqs > 0 && shape_of(d, true, &N, &mc)) {
    const size_t v = make_plan(d, backward != 0, N, mc).total;
    if (v > best) best = v;
  }
  return best;
}

kda_status kda_fwd(const kda_desc* d, const void* q, const void* k, const void* v, const void* log_alpha,
                   const void* beta, const float* init_state, void* out, float* final_state,
                   const int32_t* cu_seqlens, void* workspace, size_t workspace_bytes, void* stream) {
  return kda::fwd_checked(d, q, k, v, log_alpha, beta, init_state, out, final_state, cu_seqlens, workspace,
                          workspace_bytes, stream, nullptr);
}

}  // extern "C"

namespace kda {
// kda_fwd's validation and dispatch; `need` (optional) receives the workspace the
// problem needs once the descriptor and shapes are valid.
kda_status fwd_checked(const kda_desc* d, const void* q, const void* k, const void* v, const void* log_alpha,
                       const void* beta, const float* init_state, void* out, float* final_state,
                       const int32_t* cu_seqlens, void* workspace, size_t workspace_bytes, void* stream,
                       size_t* need) {
  if (need) *need = 0;
  if (!d) return KDA_ERROR_INVALID_VALUE;
  if (!dims_ok(d)) return KDA_ERROR_NOT_SUPPORTED;
  int N, mc;
  if (!shape_of(d, cu_seqlens != nullptr, &N, &mc)) return KDA_ERROR_INVALID_VALUE;
  if (!std::isfinite(d->scale)) return KDA_ERROR_INVALID_VALUE;
  const bool any_tok = (long long)d->B * d->T > 0;
  if (any_tok && (!q || !k || !v || !log_alpha || !beta || !out)) return KDA_ERROR_INVALID_VALUE;
  const void* al16[] = {q, k, v, log_alpha, out, init_state, final_state, workspace};
  for (const void* p : al16)
    if (p && !aligned16(p)) return KDA_ERROR_MISALIGNED;
  if (beta && ((uintptr_t)beta % (d->dtype == KDA_BF16 ? 2 : 4))) return KDA_ERROR_MISALIGNED;
  if (out && ((uintptr_t)out % (d->out_dtype == KDA_BF16 ? 2 : 4))) return KDA_ERROR_MISALIGNED;
  if (cu_seqlens && ((uintptr_t)cu_seqlens & 3u)) return KDA_ERROR_MISALIGNED;
  if (d->flags & ~(KDA_FLAG_SAVE_FOR_BACKWARD | KDA_PREP_FLAGS)) return KDA_ERROR_INVALID_VALUE;
  const bool save = (d->flags & KDA_FLAG_SAVE_FOR_BACKWARD) != 0;
  if (save && d->dtype == KDA_F32 && d->dk == 128) return KDA_ERROR_NOT_SUPPORTED;  // no fp32 backward at dk = 128
  const Plan p = make_plan(d, save, N, mc);
  if (need) *need = p.total;
  if (!workspace || workspace_bytes < p.total) return KDA_ERROR_WORKSPACE_TOO_SMALL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (cu_seqlens && env_int("KDA_DEBUG", 0) && !cu_ok(cu_seqlens, N, d->T, st)) return KDA_ERROR_INVALID_VALUE;

  Args a;
  base_args(a, d, N, mc);
  a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.beta = beta;
  a.init = init_state; a.cu = cu_seqlens;
  a.out = out; a.final_state = final_state;
  fill_ws(a, p, workspace);
  (void)hipGetLastError();  // clear a stale error so it is not blamed on this call
  clear_error();
  return launch_status(run_fwd(d, a, st));
}

void set_error(const char* msg) { std::snprintf(tl_error, sizeof tl_error, "%s", msg); }
}  // namespace kda

extern "C" {

kda_status kda_bwd(const kda_desc* d, const void* q, const void* k, const void* v, const void* log_alpha,
                   const void* beta, const float* init_state, const int32_t* cu_seqlens, const void* d_out,
                   const float* d_final_state, void* dq, void* dk, void* dv, void* dlog_alpha, void* dbeta,
                   float* d_init_state, void* workspace, size_t workspace_bytes, void* stream) {
  if (!d) return KDA_ERROR_INVALID_VALUE;
  if (!dims_ok(d)) return KDA_ERROR_NOT_SUPPORTED;
  int N, mc;
  if (!shape_of(d, cu_seqlens != nullptr, &N, &mc)) return KDA_ERROR_INVALID_VALUE;
  if (!std::isfinite(d->scale)) return KDA_ERROR_INVALID_VALUE;
  const bool any_tok = (long long)d->B * d->T > 0;
  if (any_tok && (!q || !k || !v || !log_alpha || !beta || !d_out || !dq || !dk || !dv || !dlog_alpha || !dbeta))
    return KDA_ERROR_INVALID_VALUE;
  const void* al16[] = {q, k, v, log_alpha, init_state, d_out, d_final_state, dq, dk, dv, dlog_alpha,
                        d_init_state, workspace};
  for (const void* p : al16)
    if (p && !aligned16(p)) return KDA_ERROR_MISALIGNED;
  const size_t es = d->dtype == KDA_BF16 ? 2 : 4, eo = d->out_dtype == KDA_BF16 ? 2 : 4;
  if ((beta && (uintptr_t)beta % es) || (dbeta && (uintptr_t)dbeta % eo)) return KDA_ERROR_MISALIGNED;
  if (cu_seqlens && ((uintptr_t)cu_seqlens & 3u)) return KDA_ERROR_MISALIGNED;
  if (d->dtype == KDA_F32 && d->dk == 128) return KDA_ERROR_NOT_SUPPORTED;  // fp32 backward: dk = 64 only
  if (d->flags & ~(KDA_FLAG_USE_SAVED | KDA_PREP_FLAGS)) return KDA_ERROR_INVALID_VALUE;
  const Plan p = make_plan(d, true, N, mc);
  if (!workspace || workspace_bytes < p.total) return KDA_ERROR_WORKSPACE_TOO_SMALL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (cu_seqlens && env_int("KDA_DEBUG", 0) && !cu_ok(cu_seqlens, N, d->T, st)) return KDA_ERROR_INVALID_VALUE;

  Args a;
  base_args(a, d, N, mc);
  a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.beta = beta;
  a.init = init_state; a.cu = cu_seqlens;
  a.dout = d_out; a.dfinal = d_final_state;
  a.dq = dq; a.dk_ = dk; a.dv_ = dv; a.dla = dlog_alpha; a.dbeta = dbeta; a.dinit = d_init_state;
  fill_ws(a, p, workspace);
  (void)hipGetLastError();
  clear_error();
  return launch_status(run_bwd(d, a, st));
}

kda_status kda_decode(const kda_desc* d, const void* q, const void* k, const void* v, const void* log_alpha,
                      const void* beta, float* state_pool, int32_t pool_size, const int32_t* state_indices,
                      const int32_t* num_commit, void* out, void* stream) {
  if (!d) return KDA_ERROR_INVALID_VALUE;
  if (!dims_ok(d)) return KDA_ERROR_NOT_SUPPORTED;
  if (d->B < 0 || d->T < 0 || d->T > KDA_DECODE_MAX_TOKENS || d->H < 1 || d->H > 65535) return KDA_ERROR_INVALID_VALUE;
  if ((long long)d->B * d->T * d->H >= (1LL << 31) || (long long)d->B * d->H >= (1LL << 31)) return KDA_ERROR_INVALID_VALUE;
  if (!std::isfinite(d->scale) || (d->flags & ~KDA_PREP_FLAGS) || pool_size < 0) return KDA_ERROR_INVALID_VALUE;
  if (d->B == 0 || d->T == 0) return KDA_SUCCESS;
  if (!q || !k || !v || !log_alpha || !beta || !out || !state_pool) return KDA_ERROR_INVALID_VALUE;
  if (!state_indices && pool_size < d->B) return KDA_ERROR_INVALID_VALUE;
  const void* al16[] = {q, k, v, log_alpha, out, state_pool};
  for (const void* p : al16)
    if (!aligned16(p)) return KDA_ERROR_MISALIGNED;
  if ((uintptr_t)beta % (d->dtype == KDA_BF16 ? 2 : 4)) return KDA_ERROR_MISALIGNED;
  if (((uintptr_t)state_indices & 3u) || ((uintptr_t)num_commit & 3u)) return KDA_ERROR_MISALIGNED;

  kda::DecodeArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.beta = beta;
  a.pool = state_pool; a.idx = state_indices; a.ncommit = num_commit; a.out = out;
  a.B = d->B; a.T = d->T; a.H = d->H; a.pool_size = pool_size;
  a.scale = d->scale != 0.f ? d->scale : 1.0f / std::sqrt((float)d->dk);
  a.qk_norm = (d->flags & KDA_FLAG_QK_L2NORM) != 0;
  a.gate_ls = (d->flags & KDA_FLAG_GATE_LOGSIGMOID) != 0;
  (void)hipGetLastError();
  clear_error();
  return launch_status(run_decode(d, a, static_cast<hipStream_t>(stream)));
}

size_t kda_conv_workspace_bytes(const kda_conv_desc* d) {
  if (!d || !conv_desc_ok(d) || d->B < 0 || d->T < 0) return 0;
  return conv_ws_bytes(d);
}

kda_status kda_conv_fwd(const kda_conv_desc* d, const void* x, const float* weight, const float* bias,
                        const float* init_state, void* y, float* final_state, const int32_t* cu_seqlens,
                        void* stream) {
  if (!d) return KDA_ERROR_INVALID_VALUE;
  if (!conv_desc_ok(d)) return KDA_ERROR_NOT_SUPPORTED;
  int N;
  if (!conv_shape(d, cu_seqlens != nullptr, &N)) return KDA_ERROR_INVALID_VALUE;
  const bool any_tok = (long long)d->B * d->T > 0;
  if (!weight || (any_tok && (!x || !y))) return KDA_ERROR_INVALID_VALUE;
  const void* al16[] = {x, y, init_state, final_state};
  for (const void* p : al16)
    if (p && !aligned16(p)) return KDA_ERROR_MISALIGNED;
  const void* al4[] = {weight, bias, cu_seqlens};
  for (const void* p : al4)
    if ((uintptr_t)p & 3u) return KDA_ERROR_MISALIGNED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (cu_seqlens && env_int("KDA_DEBUG", 0) && !cu_ok(cu_seqlens, N, d->T, st)) return KDA_ERROR_INVALID_VALUE;
  kda::ConvArgs c;
  conv_args(c, d, N);
  c.x = x; c.weight = weight; c.bias = bias; c.init = init_state; c.cu = cu_seqlens;
  c.y = y; c.final_state = final_state;
  (void)hipGetLastError();
  clear_error();
  return launch_status(run_conv(d, c, ConvOp::Fwd, st));
}

kda_status kda_conv_bwd(const kda_conv_desc* d, const void* x, const float* weight, const float* bias,
                        const float* init_state, const int32_t* cu_seqlens, const void* dy,
                        const float* d_final_state, void* dx, float* dweight, float* dbias,
                        float* d_init_state, void* workspace, size_t workspace_bytes, void* stream) {
  if (!d) return KDA_ERROR_INVALID_VALUE;
  if (!conv_desc_ok(d)) return KDA_ERROR_NOT_SUPPORTED;
  int N;
  if (!conv_shape(d, cu_seqlens != nullptr, &N)) return KDA_ERROR_INVALID_VALUE;
  const bool any_tok = (long long)d->B * d->T > 0;
  if (!weight || !dweight || (any_tok && (!x || !dy || !dx))) return KDA_ERROR_INVALID_VALUE;
  const void* al16[] = {x, dy, dx, init_state, d_final_state, d_init_state, workspace};
  for (const void* p : al16)
    if (p && !aligned16(p)) return KDA_ERROR_MISALIGNED;
  const void* al4[] = {weight, bias, dweight, dbias, cu_seqlens};
  for (const void* p : al4)
    if ((uintptr_t)p & 3u) return KDA_ERROR_MISALIGNED;
  const size_t need = conv_ws_bytes(d);
  if (need && (!workspace || workspace_bytes < need)) return KDA_ERROR_WORKSPACE_TOO_SMALL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (cu_seqlens && env_int("KDA_DEBUG", 0) && !cu_ok(cu_seqlens, N, d->T, st)) return KDA_ERROR_INVALID_VALUE;
  kda::ConvArgs c;
  conv_args(c, d, N);
  c.x = x; c.weight = weight; c.bias = bias; c.init = init_state; c.cu = cu_seqlens;
  c.dy = dy; c.dfinal = d_final_state; c.dx = dx;
  c.dweight = dweight; c.dbias = dbias; c.dinit = d_init_state;
  c.part = static_cast<float*>(workspace);
  (void)hipGetLastError();
  clear_error();
  return launch_status(run_conv(d, c, ConvOp::Bwd, st));
}

kda_status kda_conv_decode(const kda_conv_desc* d, const void* x, const float* weight, const float* bias,
                           float* state_pool, int32_t pool_size, const int32_t* state_indices,
                           const int32_t* num_commit, void* y, void* stream) {
  if (!d) return KDA_ERROR_INVALID_VALUE;
  if (!conv_desc_ok(d)) return KDA_ERROR_NOT_SUPPORTED;
  if (d->B < 0 || d->T < 0 || d->B > 65535 || pool_size < 0) return KDA_ERROR_INVALID_VALUE;
  if ((long long)d->B * d->T * d->D >= (1LL << 40)) return KDA_ERROR_INVALID_VALUE;
  if (d->B == 0) return KDA_SUCCESS;
  if (!weight || !state_pool || (d->T > 0 && (!x || !y))) return KDA_ERROR_INVALID_VALUE;
  if (!state_indices && pool_size < d->B) return KDA_ERROR_INVALID_VALUE;
  const void* al16[] = {x, y, state_pool};
  for (const void* p : al16)
    if (p && !aligned16(p)) return KDA_ERROR_MISALIGNED;
  const void* al4[] = {weight, bias, state_indices, num_commit};
  for (const void* p : al4)
    if ((uintptr_t)p & 3u) return KDA_ERROR_MISALIGNED;
  kda::ConvArgs c;
  std::memset(&c, 0, sizeof c);
  c.B = d->B; c.T = d->T; c.D = d->D; c.tokens = d->B * d->T;
  c.silu = d->activation == KDA_CONV_SILU;
  c.x = x; c.weight = weight; c.bias = bias; c.y = y;
  c.pool = state_pool; c.pool_size = pool_size; c.idx = state_indices; c.ncommit = num_commit;
  (void)hipGetLastError();
  clear_error();
  return launch_status(run_conv(d, c, ConvOp::Decode, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
