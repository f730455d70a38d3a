// The tuned attention shape -- fp16 storage, head_dim 128, 4 query heads per
// KV head (the Llama-3-8B layer) -- and the vector types of its kernels.
#pragma once

#include "pkv_internal.h"

namespace pkv {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;  // head dim
constexpr int kG = 4;    // query heads per KV head

}  // namespace pkv
