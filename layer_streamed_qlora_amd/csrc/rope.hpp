// The inverse rotary rotation of the backward, shared by the kernels that apply it so
// that they round alike.
//
// The forward rotates each pair (x_i, x_{i + hd/2}) of a q or k head by the angle of the
// row's position ("Fine-Tuning an 8B Parameter Model on a 4 GB Laptop GPU": the decoder
// layer is the Llama-3.1-8B one, rotary positions on q and k); the gradient goes back
// through the transposed rotation: (g1 c + g2 s, g2 c - g1 s) for the pair's (c, s).
#pragma once
#include <hip/hip_runtime.h>

namespace lsq {

// g1 at column i of a head, g2 at column i + hd/2, cs = (cos, sin) of the pair's angle;
// one fused multiply-add per output, with the other product rounded first
__device__ __forceinline__ float2 rope_inverse(float g1, float g2, float2 cs) {
  return make_float2(__builtin_fmaf(g1, cs.x, g2 * cs.y), __builtin_fmaf(g2, cs.x, -(g1 * cs.y)));
}

}  // namespace lsq
