// kda_internal.hpp -- host/device argument block and launcher declarations.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda_common.hpp"

namespace kda {

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
  void *wsW, *wsKhT, *wsQt, *wsUt, *wsAqk, *wsT;  // per (chunk, head) blocks, see WsBlock
  float* wsGam;
  void* wsS;                // backward: state at each chunk start, E [DV][DK] per chunk-head
  void* wsdS;               // backward: gradient of the state at each chunk end, E [DV][DK]
  void* wsdU;               // backward: dU, E [CH][DV]
  float* wsdQS;             // backward: scale * dO S^T, float [CH][DK]
  float* wsdKh;             // backward: U dS'^T, float [CH][DK]
  void* wsdW;               // backward: -dU S^T, E [CH][DK]
  void* wsdAqk;             // backward: scale * tril(dO U^T), E [CH][CH]
  float* wsdGam;            // backward: rowsum(dS' * S), float [DK]
  int dvs;                  // value-column slice width of the sequential passes
  int out_bf16;             // outputs and gradients stored as bf16 (else fp32)
};

hipError_t launch_chunk_map(const Args& a, hipStream_t st);
template <typename E, typename O, int DK, int DV> hipError_t launch_fwd(const Args& a, hipStream_t st);
template <typename E, int DK, int DV> hipError_t launch_bwd_front(const Args& a, hipStream_t st);
template <typename E, int DK, int DV> hipError_t launch_bwd(const Args& a, hipStream_t st);

}  // namespace kda
