// la_poly_grad.h -- host entry points of the gradient of the causal forward
// with the degree-2 polynomial kernel (la_poly_grad.hip).
#pragma once

#include "la_internal.h"

namespace la {

// Workspace of launch_poly_backward (bytes); esize: bytes per element of
// the inputs.
size_t poly_backward_workspace_bytes(int64_t BH, int64_t N, int64_t D, int64_t M, size_t esize);

// dq, dk, dv: gradients of sum(dout * out) for the causal polynomial forward,
// D, M in {32, 64}; dt 0 = fp32, 1 = bf16 (inputs and outputs).
hipError_t launch_poly_backward(int dt, const void *q, const void *k, const void *v, const void *dout, void *dq,
                                void *dk, void *dv, int64_t BH, int64_t N, int64_t D, int64_t M, void *ws,
                                hipStream_t s);

} // namespace la
