// SwiGLU backward arithmetic shared by the kernels that compute it (one
// definition, so that they round alike): with sigma(g) = 1 / (1 + e^-g),
//   h = silu(g) u = g sigma(g) u,   d gate = dh u silu'(g),
//   silu'(g) = sigma(g) (1 + g (1 - sigma(g))),   d up = dh silu(g),
// in fp32 with the hardware exp2 and reciprocal.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_bf16.h"

namespace mx {

struct Grad {
    float dg, du, h;
};

__device__ __forceinline__ Grad swiglu_grad(float g, float u, float d) {
    const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504088896341f));
    const float s = g * sig;
    const float ds = sig * (1.0f + g * (1.0f - sig));
    return Grad{d * u * ds, d * s, s * u};
}

}  // namespace mx
