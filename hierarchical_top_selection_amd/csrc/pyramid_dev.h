// pyramid_dev.h - the two pooling rules of the key pyramid, shared by the prefill
// build and the decode update so that both produce bit-identical summaries.
//
// Method steps (first step) of "Block Sparse Attention with Log-Linear
// Complexity": a leaf summarises C = 64 raw keys by their mean, and each node
// above is the mean of its g = 2 children; a node with a single child (the
// right edge of a level) is that child.
#pragma once

#include "pisa_device.h"

namespace pisa {

// Mean of column c over keys [first, first + cnt): float32 sum in key order, then / cnt.
// Keys are loaded eight at a time (independent loads in flight); the additions keep key order.
template <typename T>
__device__ inline float leaf_mean_column(const T* base, int64_t stride_t, int64_t first, int cnt,
                                         int c) {
  float s = 0.f;
  int r = 0;
  for (; r + 8 <= cnt; r += 8) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = to_f32(base[(first + r + i) * stride_t + c]);
#pragma unroll
    for (int i = 0; i < 8; ++i) s += x[i];
  }
  for (; r < cnt; ++r) s += to_f32(base[(first + r) * stride_t + c]);
  return s / (float)cnt;
}

// Unweighted mean of one or two children.
__device__ inline float node_mean(float c0, float c1, bool has_second) {
  return has_second ? (c0 + c1) * 0.5f : c0;
}

}  // namespace pisa
