// Shared between the vanilla Markov sampler and the gated / recurrent heads:
// the per-row argmax key slots of a sampling step, and host entries that
// launch one step of the Markov product when each row's rank-r row is
// already in a buffer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace dspark {

// Per-row argmax keys are folded with device-scope atomics, which MI355X
// executes at the memory side; thousands of them on the same few cache
// lines serialise.  Each row therefore has kKeyReplicas slots, each replica
// in its own 4 KB-aligned region: workgroup w folds into replica w % 16 and
// readers take the maximum over the replicas.
constexpr int kKeyReplicas = 16;
__host__ __device__ __forceinline__ int64_t replica_stride(int R) {  // in 64-bit keys
  return ((int64_t)R * 8 + 4095) / 4096 * 512;
}
__host__ __device__ __forceinline__ int64_t keys_per_step(int R) { return kKeyReplicas * replica_stride(R); }


__device__ __forceinline__ uint64_t read_key(const uint64_t* keys, int row, int R) {
  uint64_t k = 0;
#pragma unroll
  for (int q = 0; q < kKeyReplicas; ++q) {
    const uint64_t x = keys[q * replica_stride(R) + row];
    k = x > k ? x : k;
  }
  return k;
}

// One step whose rank-r rows come from ebuf ([R, gamma, r] float32): the
// step's logits base[:, step] + E @ W2 (c * tanh(l / c) when softcap c > 0,
// then greedy), the argmax (or Gumbel-max at 1 / invT) folded into keys_out.
// W2 is [r, V] in wdtype.  Returns the launch status.
hipError_t markov_step_embedded(const float* base, const float* ebuf, const void* w2, int wdtype,
                                uint64_t* keys_out, float* step_logits, int R, int gamma, int V, int r, int step,
                                float softcap, float temperature, uint64_t seed, hipStream_t s);
// Zero n key slots (a fill kernel: safe under stream capture).
hipError_t markov_zero_keys(uint64_t* keys, int64_t n, hipStream_t s);
// The whole gamma-step sampler in one persistent cooperative launch, with W2
// held in registers across the steps (bf16 weights, R <= 128 rows, r a
// multiple of 32 up to 256, V a multiple of 8, 16-byte aligned buffers).
// keys: gamma * keys_per_step(R) zeroed slots; tokens [R, gamma] are written
// directly.  hipErrorNotSupported (nothing enqueued) when the shape or the
// device does not allow it.
bool markov_round_eligible(int R, int gamma, int V, int r, const void* base, const void* w1, const void* w2,
                           const void* step_logits);
hipError_t markov_round_launch(const float* base, const uint16_t* w1, const uint16_t* w2, const int32_t* first_prev,
                               int32_t* tokens, float* step_logits, int R, int gamma, int V, int r, float invT,
                               int greedy, uint32_t slo, uint32_t shi, uint64_t* keys, uint32_t spin_limit,
                               int32_t* status, hipStream_t s);
// Teacher-forced logits of N rows (one step each, prev from the caller) with W2 held in registers:
// logits [N, V] (soft-capped when softcap > 0) and each row's argmax folded into the zeroed key
// slots of keys_per_step(N).  Same shape limits as the round kernel (any N >= 1).
// hipErrorNotSupported (nothing enqueued) when the shape or the device does not allow it.
bool markov_rows_eligible(int N, int V, int r, const void* base, const void* w1, const void* w2, const void* logits);
hipError_t markov_rows_launch(const float* base, const uint16_t* w1, const uint16_t* w2, const int32_t* prev,
                              float* logits, int N, int V, int r, float softcap, uint64_t* keys, int32_t* status,
                              hipStream_t s);
// Poll limit of the bounded waits inside cooperative grids (dspark_set_wait_limit).
uint32_t wait_limit();
// tokens[row, step] = the argmax index folded in step's keys, for R x gamma.
hipError_t markov_finalize_tokens(const uint64_t* keys, int32_t* tokens, int R, int gamma, int V,
                                  int32_t* status, hipStream_t s);

}  // namespace dspark
