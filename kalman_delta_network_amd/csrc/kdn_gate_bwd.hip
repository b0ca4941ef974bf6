// Backward of the gated layer: gradients with respect to the gate
// pre-activations ("Kalman Delta Networks: Uncertainty-aware Associative
// Memory", summary page, method step 1: alpha = sigmoid(z), omega =
// softplus(z), r = r_min + softplus(z)).
//
// The step also normalises q and k per token-head, x_hat = x / max(|x|, eps).
//
// The diagonal bf16 form runs the chunked adjoint on the raw inputs: its
// kernels form the gates and the normalised rows as the gated forward does,
// and take the gates' derivatives where they write the gradients.  Other
// forms, and pairs outside the chunked range, run the fp32 adjoint of
// kdn_backward.hip on the prologue's values: one pass widens v and dO to
// fp32, normalises the q and k rows and evaluates the gates into the
// workspace (the same fp32 functions as the gated forward), the adjoint runs
// on them, and a pass takes the gates' derivatives.  Last, one pass over the
// q and k rows applies the normalisation's Jacobian.  The chain rule:
//   d x = (d x_hat - x_hat (x_hat . d x_hat)) / |x|   (d x_hat / eps where
//         |x| < eps: the map is then x / eps),
//   d z_alpha = d alpha * sigmoid(z) sigmoid(-z),
//   d z_omega = d omega * sigmoid(z),   d z_r = d r * sigmoid(z).
#include "kdn_gates.h"
#include "kdn_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>

namespace kdn {
namespace {

enum GateOp { kCopy = 0, kSigmoid = 1, kSoftplus = 2, kRSoftplus = 3 };

__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// Only the (batch, head) pairs flagged in `only` (when given) need the fp32
// copies: element i of a [B, T, H, width] array belongs to pair
// (i / width / (T H)) H + (i / width) % H.
struct PairFilter {
    const int* only;
    size_t TH;
    int H, width, units;
    __device__ __forceinline__ bool skip(size_t i) const {
        if (!only) return false;
        const size_t row = i / size_t(width);
        return !only[(row / TH) * size_t(H) + row % size_t(H)];
    }
    // no pair flagged (the usual case): the whole workgroup has nothing to do
    __device__ __forceinline__ bool none() const {
        if (!only) return false;
        __shared__ int any;
        if (threadIdx.x == 0) any = 0;
        __syncthreads();
        for (int u = threadIdx.x; u < units; u += blockDim.x)
            if (only[u]) any = 1;
        __syncthreads();
        return any == 0;
    }
};

// y[i] = op(x[i]) in fp32
template <typename Tin>
__global__ void __launch_bounds__(256) gate_forward_kernel(const Tin* __restrict__ x, float* __restrict__ y,
                                                           size_t n, int op, PairFilter pf) {
    if (pf.none()) return;
    const size_t stride = size_t(gridDim.x) * blockDim.x;
    for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        if (pf.skip(i)) continue;
        const float z = widen(x[i]);
        float out = z;
        if (op == kSigmoid) out = gate_sigmoid(z);
        else if (op == kSoftplus) out = gate_softplus(z);
        else if (op == kRSoftplus) out = kGateRMin + gate_softplus(z);
        y[i] = out;
    }
}

// d[i] *= the derivative of the gate at z[i]
template <typename Tin>
__global__ void __launch_bounds__(256) gate_grad_kernel(const Tin* __restrict__ z, float* __restrict__ d, size_t n,
                                                        int op, PairFilter pf) {
    if (pf.none()) return;
    const size_t stride = size_t(gridDim.x) * blockDim.x;
    for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        if (pf.skip(i)) continue;
        const float x = widen(z[i]);
        // sigmoid' = sigmoid(z) sigmoid(-z) (no cancellation in 1 - sigmoid);
        // softplus' = sigmoid
        const float g = op == kSigmoid ? gate_sigmoid(x) * gate_sigmoid(-x) : gate_sigmoid(x);
        d[i] *= g;
    }
}

// |x|^2 of row `row` (dk channels), in every lane of the calling wave
template <typename Tin>
__device__ __forceinline__ float row_sumsq(const Tin* __restrict__ x, size_t row, int dk) {
    const int lane = threadIdx.x & 63;
    float s = 0.f;
    for (int i = lane; i < dk; i += 64) {
        const float v = widen(x[row * dk + i]);
        s = fmaf(v, v, s);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    return s;
}

// y = x / max(|x|, eps) per row of dk channels (one wave per row)
template <typename Tin>
__global__ void __launch_bounds__(256) row_normalize_kernel(const Tin* __restrict__ x, float* __restrict__ y,
                                                            size_t rows, int dk, PairFilter pf) {
    if (pf.none()) return;
    const int lane = threadIdx.x & 63;
    const size_t waves = size_t(gridDim.x) * (blockDim.x / 64);
    for (size_t row = size_t(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6); row < rows; row += waves) {
        if (pf.skip(row)) continue;  // (width 1: one row per token-head)
        const float inv = inv_norm(row_sumsq(x, row, dk));
        for (int i = lane; i < dk; i += 64) y[row * dk + i] = widen(x[row * dk + i]) * inv;
    }
}

// d <- the gradient of the raw rows x given d = the gradient of their
// normalised rows (one wave per row)
template <typename Tin>
__global__ void __launch_bounds__(256) row_normalize_grad_kernel(const Tin* __restrict__ x, float* __restrict__ d,
                                                                 size_t rows, int dk) {
    const int lane = threadIdx.x & 63;
    const size_t waves = size_t(gridDim.x) * (blockDim.x / 64);
    for (size_t row = size_t(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6); row < rows; row += waves) {
        const float nrm = sqrtf(row_sumsq(x, row, dk));
        const bool floored = !(nrm >= kNormEps);
        const float inv = 1.f / (floored ? kNormEps : nrm);
        float proj = 0.f;  // x_hat . d
        for (int i = lane; i < dk; i += 64) proj = fmaf(widen(x[row * dk + i]) * inv, d[row * dk + i], proj);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) proj += __shfl_xor(proj, off, 64);
        if (floored) proj = 0.f;
        for (int i = lane; i < dk; i += 64) {
            const size_t e = row * dk + i;
            d[e] = (d[e] - widen(x[e]) * inv * proj) * inv;
        }
    }
}

// Four consecutive channels as fp32 (8-byte bf16 or 16-byte fp32 load)
__device__ __forceinline__ float4 load4(const uint16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                       __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// sum over the LPR lanes of a row (aligned groups of LPR lanes)
template <int LPR>
__device__ __forceinline__ float group_sum(float s) {
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    return s;
}

// The same map as row_normalize_grad_kernel for the q rows (blockIdx.y 0)
// and the k rows (blockIdx.y 1) in one launch: LPR = dk / 4 lanes per row,
// four channels per lane, each element read and written once.
template <typename Tin, int LPR>
__global__ void __launch_bounds__(256) row_normalize_grad4_kernel(const Tin* __restrict__ xq,
                                                                  const Tin* __restrict__ xk, float* __restrict__ dq,
                                                                  float* __restrict__ dk, size_t rows) {
    constexpr int DK = 4 * LPR;
    constexpr int RPB = 256 / LPR;  // rows per workgroup and iteration
    const Tin* __restrict__ x = blockIdx.y ? xk : xq;
    float* __restrict__ d = blockIdx.y ? dk : dq;
    const int sub = int(threadIdx.x) % LPR;
    const size_t stride = size_t(gridDim.x) * RPB;
    // the LPR lanes of a row share it, so they take the loop together
    for (size_t row = size_t(blockIdx.x) * RPB + threadIdx.x / LPR; row < rows; row += stride) {
        const size_t e = row * DK + 4 * sub;
        const float4 v = load4(x + e);
        float4 g = *reinterpret_cast<const float4*>(d + e);
        float s = v.x * v.x;
        s = fmaf(v.y, v.y, s);
        s = fmaf(v.z, v.z, s);
        s = fmaf(v.w, v.w, s);
        const float nrm = sqrtf(group_sum<LPR>(s));
        const bool floored = !(nrm >= kNormEps);
        const float inv = 1.f / (floored ? kNormEps : nrm);
        float proj = (v.x * inv) * g.x;  // x_hat . d
        proj = fmaf(v.y * inv, g.y, proj);
        proj = fmaf(v.z * inv, g.z, proj);
        proj = fmaf(v.w * inv, g.w, proj);
        proj = group_sum<LPR>(proj);
        if (floored) proj = 0.f;
        g.x = (g.x - v.x * inv * proj) * inv;
        g.y = (g.y - v.y * inv * proj) * inv;
        g.z = (g.z - v.z * inv * proj) * inv;
        g.w = (g.w - v.w * inv * proj) * inv;
        *reinterpret_cast<float4*>(d + e) = g;
    }
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

struct GatedSizes {
    size_t nk, nv, na, nw, nr;
};

GatedSizes gated_sizes(int variant, int B, int T, int H, int dk, int dv) {
    const size_t toks = size_t(B) * size_t(T) * size_t(H);
    const bool iso = variant == 1 || variant == 2, chan = variant != 1;
    return {toks * dk, toks * dv, chan ? toks * dk : toks, iso ? toks : toks * dk, toks};
}

// bytes of the fp32 copies (each rounded up to 256)
size_t copies_bytes(const GatedSizes& n) {
    const size_t f = sizeof(float);
    return 2 * round256(n.nk * f) + 2 * round256(n.nv * f) + round256(n.na * f) + round256(n.nw * f) +
           round256(n.nr * f);
}

template <typename Tin>
hipError_t run(const BwdArgs& a, hipStream_t s) {
    const GatedSizes n = gated_sizes(a.variant, a.B, a.T, a.H, a.dk, a.dv);
    // the adjoint's workspace, then the fp32 copies at the workspace's end
    // (16-byte aligned): the adjoint takes everything before them
    const uintptr_t end = reinterpret_cast<uintptr_t>(a.work) + a.work_bytes;
    char* w = reinterpret_cast<char*>((end - copies_bytes(n)) & ~uintptr_t(15));
    const size_t base = size_t(w - reinterpret_cast<char*>(a.work));
    auto take = [&](size_t count) {
        float* p = reinterpret_cast<float*>(w);
        w += round256(count * sizeof(float));
        return p;
    };
    float* fq = take(n.nk);
    float* fk = take(n.nk);
    float* fv = take(n.nv);
    float* fa = take(n.na);
    float* fw = take(n.nw);
    float* fr = take(n.nr);
    float* fdo = take(n.nv);
    // The diagonal bf16 form takes the chunked path on the raw inputs (its
    // kernels form the gated values as the gated forward does); the fp32
    // copies then serve only the pairs outside its range, which its
    // checkpoint sweep flags.
    BwdArgs c = a;
    c.gates = true;
    c.work_bytes = base;
    const bool chunked = backward_chunked_eligible(c);
    hipError_t e = hipSuccess;
    PairFilter pf{nullptr, size_t(a.T) * size_t(a.H), a.H, 1, a.B * a.H};
    if (chunked) {
        e = launch_backward_chunked_main(c, s);
        if (e != hipSuccess) return e;
        pf.only = backward_chunk_flags(c);
    }
    const auto fwd = [&](const void* x, float* y, size_t count, int op, int width) {
        if (count == 0) return;
        const unsigned blocks = unsigned(count / 256 + 1 < 8192 ? count / 256 + 1 : 8192);
        PairFilter f = pf;
        f.width = width;
        hipLaunchKernelGGL(gate_forward_kernel<Tin>, dim3(blocks), dim3(256), 0, s, static_cast<const Tin*>(x), y,
                           count, op, f);
    };
    const size_t rows = size_t(a.B) * size_t(a.T) * size_t(a.H);
    const unsigned row_blocks = unsigned(rows / 4 + 1 < 8192 ? rows / 4 + 1 : 8192);  // 4 rows per block
    if (rows) {
        hipLaunchKernelGGL(row_normalize_kernel<Tin>, dim3(row_blocks), dim3(256), 0, s, static_cast<const Tin*>(a.q),
                           fq, rows, a.dk, pf);
        hipLaunchKernelGGL(row_normalize_kernel<Tin>, dim3(row_blocks), dim3(256), 0, s, static_cast<const Tin*>(a.k),
                           fk, rows, a.dk, pf);
    }
    const int wa = int(n.na / (rows ? rows : 1)), ww = int(n.nw / (rows ? rows : 1));  // per-token widths
    fwd(a.v, fv, n.nv, kCopy, a.dv);
    fwd(a.alpha, fa, n.na, kSigmoid, wa);
    fwd(a.omega, fw, n.nw, kSoftplus, ww);
    fwd(a.r, fr, n.nr, kRSoftplus, 1);
    if (a.dO) fwd(a.dO, fdo, n.nv, kCopy, a.dv);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    BwdArgs f = a;
    f.work_bytes = base;
    f.q = fq;
    f.k = fk;
    f.v = fv;
    f.alpha = fa;
    f.omega = fw;
    f.r = fr;
    f.dO = a.dO ? fdo : nullptr;
    f.dtype = 0;  // the token path runs on the fp32 copies
    if (chunked) e = launch_backward_chunked_fallback(c, f, s);
    else e = launch_backward(f, s);
    if (e != hipSuccess) return e;
    // The chunked kernels leave the gradients of the gate pre-activations
    // themselves; the token path's (all pairs, or only the flagged ones)
    // still take the gates' derivatives here.
    const auto grad = [&](const void* z, float* d, size_t count, int op, int width) {
        if (count == 0) return;
        const unsigned blocks = unsigned(count / 256 + 1 < 8192 ? count / 256 + 1 : 8192);
        PairFilter f = pf;
        f.width = width;
        hipLaunchKernelGGL(gate_grad_kernel<Tin>, dim3(blocks), dim3(256), 0, s, static_cast<const Tin*>(z), d,
                           count, op, f);
    };
    if (rows) {
        const bool vec = (a.dk == 64 || a.dk == 128) && aligned16(a.q) && aligned16(a.k) && aligned16(a.dq) &&
                         aligned16(a.dk_);
        if (vec) {
            const size_t rpb = size_t(256 / (a.dk / 4));
            const unsigned blocks = unsigned(std::min<size_t>((rows + rpb - 1) / rpb, 4096));
            if (a.dk == 128)
                hipLaunchKernelGGL((row_normalize_grad4_kernel<Tin, 32>), dim3(blocks, 2), dim3(256), 0, s,
                                   static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k), a.dq, a.dk_, rows);
            else
                hipLaunchKernelGGL((row_normalize_grad4_kernel<Tin, 16>), dim3(blocks, 2), dim3(256), 0, s,
                                   static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k), a.dq, a.dk_, rows);
        } else {
            hipLaunchKernelGGL(row_normalize_grad_kernel<Tin>, dim3(row_blocks), dim3(256), 0, s,
                               static_cast<const Tin*>(a.q), a.dq, rows, a.dk);
            hipLaunchKernelGGL(row_normalize_grad_kernel<Tin>, dim3(row_blocks), dim3(256), 0, s,
                               static_cast<const Tin*>(a.k), a.dk_, rows, a.dk);
        }
    }
    grad(a.alpha, a.dalpha, n.na, kSigmoid, wa);
    grad(a.omega, a.domega, n.nw, kSoftplus, ww);
    grad(a.r, a.dr, n.nr, kSoftplus, 1);
    return hipGetLastError();
}

}  // namespace

size_t backward_gated_workspace_bytes(int variant, int B, int T, int H, int dk, int dv) {
    const size_t base = backward_workspace_bytes(B, T, H, dk, dv);
    if (base == 0) return 0;
    return round256(base) + copies_bytes(gated_sizes(variant, B, T, H, dk, dv));
}

size_t backward_gated_workspace_bytes_for(int variant, int dtype, int B, int T, int H, int dk, int dv) {
    const size_t base = backward_workspace_bytes_for(variant, dtype, B, T, H, dk, dv);
    if (base == 0) return 0;
    return round256(base) + copies_bytes(gated_sizes(variant, B, T, H, dk, dv));
}

hipError_t launch_backward_gated(const BwdArgs& a, hipStream_t stream) {
    if (a.variant == 3) return hipErrorNotSupported;  // no gate step with grouped noise
    return a.dtype == 1 ? run<uint16_t>(a, stream) : run<float>(a, stream);
}

}  // namespace kdn
