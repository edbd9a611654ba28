// kda_conv.hpp -- argument block and launchers of the short causal convolution
// (kda_conv_fwd, kda_conv_bwd, kda_conv_decode).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Short causal convolution with a carried state (kda_conv_fwd, kda_conv_bwd,
// kda_conv_decode).
constexpr int CONV_BWD_TILE = 256;     // tokens per backward tile (one row of partial sums)
struct ConvArgs {
  int B, T, D, N;                      // rows, tokens per row, channels, sequences
  int tokens;                          // B * T
  int silu;                            // 1: y = z * sigmoid(z), 0: y = z
  const void* x;                       // [tokens][D] (decode: [B][T][D]) in the input dtype
  const float* weight;                 // [D][W]
  const float* bias;                   // [D] or null
  const float* init;                   // [N][W-1][D] or null (zero)
  const int32_t* cu;                   // [N + 1] or null: N = B rows of T tokens
  void* y;                             // like x, in the output dtype
  float* final_state;                  // [N][W-1][D] or null
  const void* dy;                      // like x
  const float* dfinal;                 // [N][W-1][D] or null (zero)
  void* dx;                            // like x, in the output dtype
  float *dweight, *dbias, *dinit;      // [D][W]; [D] or null; [N][W-1][D] or null
  float* part;                         // workspace: [tiles][W+1][D] partial sums
  float* pool;                         // decode: [pool_size][W-1][D], updated in place
  const int32_t *idx, *ncommit;        // decode: [B] slots (null: b); [B] committed tokens (null: T)
  int pool_size;
};

template <typename E, typename O, int W> hipError_t launch_conv_fwd(const ConvArgs& c, hipStream_t st);
template <typename E, typename O, int W> hipError_t launch_conv_bwd(const ConvArgs& c, hipStream_t st);
template <typename E, typename O, int W> hipError_t launch_conv_decode(const ConvArgs& c, hipStream_t st);

}  // namespace kda
