// kda_internal.hpp -- host/device argument block and launcher declarations.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"
#include "kda_common.hpp"

namespace kda {

constexpr int GS_PARTS = 2048;   // work-groups of the gradient-scale pre-pass (one partial maximum each)

struct Args {
  // problem
  int B, T, H, dk, dv, N;   // N = number of sequences
  int max_chunks;           // chunk slots (upper bound on the real chunk count)
  float scale;
  // inputs
  const void *q, *k, *v, *la, *beta;
  const float* init;
  const int32_t* cu;        // may be null: N = B sequences of T tokens
  // forward outputs
  void* out;
  float* final_state;
  // backward inputs / outputs
  const void* dout;
  const float* dfinal;
  void *dq, *dk_, *dv_, *dla, *dbeta;
  float* dinit;
  // workspace
  ChunkInfo* chunks;        // [max_chunks]
  int32_t* seq_chunk0;      // [N + 1]
  int32_t* seq_order;       // [N] sequences by decreasing chunk count
  void *wsW, *wsKhT, *wsQt, *wsUt, *wsAqk, *wsT;  // per (chunk, head) blocks, see WsBlock
  float* wsGam;
  int32_t* steep;           // [chunk slots * H] 1 where the chunk-head takes the 8-token-group path
  // backward only (per chunk-head blocks; see WsBlock for shapes and types)
  float* wsUtF;             // U~^T in fp32 [DV][CH] (the backward's state pass reads it)
  float* wsG;               // un-beta strict Gram K+ K-^T
  float* wsKhF;             // Kh token-major: fp32, or a split pair of fp16 arrays (bf16 inputs)
  void* wsKhTL;             // bf16 inputs: lo half of Kh^T (Kh^T itself is then the hi half)
  float* wsS;               // state entering each chunk, fp32 [DK][DV]
  float* wsU;               // U, fp32 [CH][DV]
  float* wsdS;              // gradient of the state leaving each chunk, fp32 [DK][DV]
  float* wsdU;              // dU, fp32 [CH][DV]
  // power-of-two scale of the upstream gradients (bf16 inputs; null otherwise):
  // gscale[0] = s multiplies dO and dS_final as the kernels read them, gscale[1] =
  // 1/s every gradient they store; gs_part holds the pre-pass's partial maxima
  float* gscale;
  float* gs_part;
  int dfinal_scaled;        // dfinal already carries s (a stretch's dS_out from the segment scan)
  int dvs;                  // value-column slice width of the sequential passes
  int out_bf16;             // outputs and gradients stored as bf16 (else fp32)
  // fused input preparation
  int qk_norm;              // q, k rows L2-normalised inside (KDA_FLAG_QK_L2NORM)
  int gate_ls;              // log_alpha holds a raw gate x; log alpha = logsigmoid(x)
  float* wsDQK;             // backward with qk_norm: dq^, dk^ (normalised-input gradients),
                            // fp32 [2][CH][DK] per chunk-head
  // segment scan of long sequences (forward): each sequence split into `segs`
  // stretches of whole chunks that run in parallel
  int segs;                 // 1: no segmentation
  int32_t* vsc0;            // [N*segs + 1] first chunk of each stretch
  int32_t* vord;            // [N*segs] stretch order (identity)
  float* seg_in;            // [N*segs][H][DK][DV] state entering each stretch
  float* seg_loc;           // [N*segs][H][DK][DV] end state of each stretch run from zero
  float* seg_m;             // [N*segs][H][DK][DK] transfer of each stretch
};

// Decode / replay step (kda_decode).
struct DecodeArgs {
  const void *q, *k, *v, *la, *beta;   // [B][T][H][.] in the input dtype
  float* pool;                         // [pool_size][H][DK][DV], updated in place
  const int32_t* idx;                  // [B] pool slot per sequence; null: slot b
  const int32_t* ncommit;              // [B] tokens whose state is committed; null: T
  void* out;                           // [B][T][H][DV] in the output dtype
  int B, T, H, pool_size;
  float scale;
  int qk_norm, gate_ls;                // fused input preparation, as in Args
};

// Opt-in per-kernel timing (kda_timing_enable): a no-op unless enabled.
void timing_begin(const char* name, hipStream_t st);
void timing_end(hipStream_t st);
void note_launch(const char* name);   // keeps the first failing launch of this call (kda_last_error)

// Bracket one launch statement with the timing hooks.
#define KDA_TIMED(name, st, launch) \
  do {                              \
    ::kda::timing_begin(name, st);  \
    launch;                         \
    ::kda::note_launch(name);       \
    ::kda::timing_end(st);          \
  } while (0)

// kda_fwd's host validation and dispatch (kda_api.cpp); `need`, when given, receives
// the workspace bytes the problem needs (0 until the descriptor and shapes pass).
kda_status fwd_checked(const kda_desc* d, const void* q, const void* k, const void* v, const void* log_alpha,
                       const void* beta, const float* init_state, void* out, float* final_state,
                       const int32_t* cu_seqlens, void* workspace, size_t workspace_bytes, void* stream,
                       size_t* need);
void set_error(const char* msg);   // the text kda_last_error returns on this host thread

hipError_t launch_chunk_map(const Args& a, hipStream_t st);
int device_cus();                  // compute units of the current device
int fwd_segments(int N, int H, int dv, long long tokens, bool save);   // stretches per sequence (segment scan)
int pick_dvs(int units, int dv);   // value-slice width of the sequential passes (bf16 inputs)
hipError_t launch_segment_map(const Args& a, hipStream_t st);   // stretches of each sequence (vsc0, vord)
template <int DK, int DV> hipError_t launch_segment_rscan(const Args& a, hipStream_t st);   // backward scan
template <typename E, typename O, int DK, int DV> hipError_t launch_fwd(const Args& a, hipStream_t st, bool save);
template <typename E, int DK, int DV> hipError_t launch_bwd_front(const Args& a, hipStream_t st);
template <typename E, typename O, int DK, int DV> hipError_t launch_bwd(const Args& a, hipStream_t st, bool saved);
template <typename E, typename O, int DK, int DV> hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);

}  // namespace kda
