// Gate step of the diagonal KDN layer, evaluated inside the forward kernels
// on pre-activations ("Kalman Delta Networks: Uncertainty-aware Associative
// Memory", summary page, method step 1): per-channel decay alpha = sigmoid(z),
// per-channel process noise omega = softplus(z), per-token observation noise
// r = r_min + softplus(z) with r_min = 0.01.
//
// fp32 on the hardware exp2 / log2 / reciprocal (v_exp_f32, v_log_f32,
// v_rcp_f32, about 1 ulp each):
//  - sigmoid(z) = 1 / (1 + 2^(-z log2 e)); for z < -88 the power is +inf and
//    the result 0 (true value below 1e-38);
//  - softplus(z) = max(z, 0) + log(1 + e) with e = 2^(-|z| log2 e) in (0, 1],
//    so nothing overflows.  log(1 + e) is ln 2 * log2(u) for u = fl(1 + e),
//    plus the rounding error of u, e - (u - 1) (both differences are exact):
//    log(u + d) = log(u) + d / u + O(d^2) and u = 1 + O(e), so adding d instead
//    of d / u errs by about d e.  The result keeps fp32 relative accuracy for
//    every z, including z << 0 where softplus(z) = e (1 - e / 2 + ...) and a
//    bare log2(fl(1 + e)) would lose every digit below 2^-24.
#pragma once

#include <hip/hip_runtime.h>

namespace kdn {

constexpr float kGateRMin = 0.01f;
// The step before the recurrence also normalises q and k per token-head:
// x / max(|x|, kNormEps) over the d_k channels (unit-norm keys, summary page,
// core method; queries alike).
constexpr float kNormEps = 1e-6f;
// 1 / max(sqrt(s), eps) = rsqrt(max(s, eps^2)) (eps^2 is a normal fp32 number)
__device__ __forceinline__ float inv_norm(float sumsq) {
    return __builtin_amdgcn_rsqf(fmaxf(sumsq, kNormEps * kNormEps));
}
constexpr float kLog2E = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float gate_sigmoid(float z) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2E * z));
}

__device__ __forceinline__ float gate_softplus(float z) {
    const float e = __builtin_amdgcn_exp2f(-kLog2E * fabsf(z));
    const float u = 1.f + e;
    const float d = e - (u - 1.f);  // rounding error of u (exact)
    return fmaf(kLn2, __builtin_amdgcn_logf(u), d + fmaxf(z, 0.f));
}

}  // namespace kdn
