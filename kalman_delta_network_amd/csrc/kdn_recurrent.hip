// kdn_recurrent.hip -- token-by-token KDN recurrence for gfx950.
//
// One workgroup owns one (batch, head) pair and keeps its whole d_k x d_v
// memory S in registers for the full sequence.  Wave w owns the 32 value
// columns [32w, 32w + 32); inside a wave, lane = (row group rg in 0..7,
// column quad cq in 0..7): the lane holds rows rg, rg + 8, ... (d_k / 8 rows)
// of 4 consecutive columns.  Every column reduction over the key dimension
// is then a reduction inside one wave (registers, then 3 lane-xor steps), so
// waves never wait for each other inside the token loop.
//
// Per token (KDN summary page, method steps 2-5; isotropic variant per the
// closing sentence of that section, with a scalar decay or, in its general
// form, one decay per key channel and the trace projection
// a = mean_i alpha_i^2 for the uncertainty scalar):
//   every wave redundantly runs the per-channel part (lane owns channels
//   lane and lane + 64): predict p_hat, gain denominator r + sum p_hat k^2,
//   kappa, kappa^T q, posterior p; it stages (alpha_i, k_i, q_i, kappa_i) in
//   its own slice of LDS;
//   then on its columns: S_hat = diag(alpha) S, the two key-dimension dot
//   products S_hat^T k and S_hat^T q in one pass, innovation
//   delta = v - S_hat^T k, readout o = S_hat^T q + (kappa^T q) delta (the
//   post-write readout expanded), and the write S = S_hat + kappa delta^T.
//
// Packed variable-length batches: unit b * H + h runs sequence b, whose
// tokens are rows [cu[b], cu[b + 1]) of the [T, H] token grid.
//
// The decode step is this kernel with T = 1 and the state updated in place:
// a barrier after the initial state loads makes every wave read p before any
// wave writes it back.
#include "kdn_gates.h"
#include "kdn_internal.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kdn {
namespace {

typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(uint32_t(x) << 16); }

__device__ __forceinline__ void from_f32(float* p, float x) { *p = x; }
__device__ __forceinline__ void from_f32(bf16_t* p, float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) {
        *p = bf16_t((u >> 16) | 0x40u);  // quiet NaN
    } else {
        u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest, ties to even
        *p = bf16_t(u >> 16);
    }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// LDS written by some lanes of a wave and read by other lanes of the same
// wave: order the accesses at wavefront scope (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
    // One wave's LDS operations execute in order, so waiting for this wave's
    // own LDS traffic and keeping the compiler from moving memory accesses
    // across is enough; a memory fence would also wait for every global load
    // still in flight (the next token's prefetch).
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// VAR: 0 diagonal, 1 isotropic, 2 isotropic with per-channel decay.
// GR (diagonal only): grouped observation noise, one r and one uncertainty
// state p per group of 64 value columns (waves 2g, 2g + 1 form group g)
template <int DK, int DV, int VAR, typename Tin, bool GR = false>
__global__ void __launch_bounds__(DV * 2)
kdn_recurrent_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                     const Tin* __restrict__ v, const Tin* __restrict__ alpha,
                     const Tin* __restrict__ omega, const Tin* __restrict__ r,
                     const float* __restrict__ c0, float mu, int T, int H, const float* S0,
                     const float* p0, Tin* __restrict__ o, float* S_T, float* p_T,
                     const int* __restrict__ cu, const int* __restrict__ ord, int nseq, int gates) {
    constexpr bool ISO = VAR != 0;       // one uncertainty scalar per head
    constexpr bool CHAN = VAR != 1;      // one decay per key channel
    constexpr int NW = DV / 32;   // waves per workgroup
    constexpr int CPL = DK / 64;  // channels per lane
    constexpr int RPT = DK / 8;   // memory rows per thread
    static_assert(DK % 64 == 0 && DV % 32 == 0, "unsupported tile");
    static_assert(!GR || VAR == 0, "grouped noise is a diagonal form");
    constexpr int NG = GR ? DV / 64 : 1;  // uncertainty groups

    __shared__ float4 chan[NW][DK];

    // block = rank * H + h; the sequence of rank `rank` is ord[rank] for a
    // packed batch with a scheduling order (longest first balances the GPU)
    const int h = int(blockIdx.x) % H;
    const int rank = int(blockIdx.x) / H;
    const size_t b = size_t(cu && ord ? min(max(ord[rank], 0), nseq - 1) : rank);
    const int unit = int(b) * H + h;  // index of the [B, H, ...] states
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int cq = lane & 7;
    const int rg = lane >> 3;
    const int col = wave * 32 + cq * 4;
    const int grp = GR ? wave / 2 : 0;  // uncertainty group of this wave's columns
    // this unit's sequence: len tokens from token-grid row tok0 on (packed
    // sequences: bounds from the offsets, clamped into the grid of T rows)
    size_t tok0 = b * size_t(T);
    int len = T;
    if (cu) {
        const int s0 = min(max(cu[b], 0), T);
        const int s1 = min(max(cu[b + 1], s0), T);
        tok0 = size_t(s0);
        len = s1 - s0;
    }

    const size_t sbase = size_t(unit) * DK * DV;
    float S[RPT][4];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + 8 * m;
        if (S0) {
            const float4 s4 = *reinterpret_cast<const float4*>(S0 + sbase + size_t(i) * DV + col);
            S[m][0] = s4.x; S[m][1] = s4.y; S[m][2] = s4.z; S[m][3] = s4.w;
        } else {
            S[m][0] = S[m][1] = S[m][2] = S[m][3] = 0.f;
        }
    }
    float p[CPL];
    float pb = 0.f;
    if (ISO) {
        pb = p0 ? p0[unit] : c0[h];
    } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) p[c] = p0 ? p0[(size_t(unit) * NG + grp) * DK + lane + 64 * c] : c0[h];
    }
    __syncthreads();  // all initial reads happen before any in-place write

    const float inv_dk = 1.0f / float(DK);
    for (int t = 0; t < len; ++t) {
        const size_t tok = (tok0 + size_t(t)) * size_t(H) + size_t(h);
        float rt = to_f32(r[GR ? tok * NG + grp : tok]);
        // gates (diagonal layer): alpha, omega and r arrive as pre-activations
        if (gates) rt = kGateRMin + gate_softplus(rt);
        float kk[CPL], qq[CPL], aa[CPL], kap[CPL];
        float mq;  // kappa^T q
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            kk[c] = to_f32(k[tok * DK + lane + 64 * c]);
            qq[c] = to_f32(q[tok * DK + lane + 64 * c]);
        }
        if (ISO) {
            // trace-projected predict b_hat = a b + omega / d_k; a = alpha^2,
            // or with per-channel decay the mean of alpha_i^2 over the channels
            float w = to_f32(omega[tok]);
            if (gates) w = gate_softplus(w);
            float a2 = 0.f, n = 0.f, kq = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                aa[c] = CHAN ? to_f32(alpha[tok * DK + lane + 64 * c]) : to_f32(alpha[tok]);
                if (gates) aa[c] = gate_sigmoid(aa[c]);
                a2 += aa[c] * aa[c];
                n += kk[c] * kk[c];
                kq += kk[c] * qq[c];
            }
            if (CHAN) a2 = wave_sum(a2) * inv_dk;
            else a2 = aa[0] * aa[0];
            const float bh = a2 * pb + w * inv_dk;
            n = wave_sum(n);
            kq = wave_sum(kq);
            const float beta = bh / (rt + bh * n);
#pragma unroll
            for (int c = 0; c < CPL; ++c) kap[c] = beta * kk[c];
            mq = beta * kq;
            pb = bh / (1.0f + (mu / (float(DK) * rt)) * n * bh);
        } else {
            float ph[CPL];
            float s = 0.f, kq = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                aa[c] = to_f32(alpha[tok * DK + lane + 64 * c]);
                float w = to_f32(omega[tok * DK + lane + 64 * c]);
                if (gates) {
                    aa[c] = gate_sigmoid(aa[c]);
                    w = gate_softplus(w);
                }
                ph[c] = aa[c] * aa[c] * p[c] + w;
                s += ph[c] * kk[c] * kk[c];
                kq += ph[c] * kk[c] * qq[c];
            }
            s = wave_sum(s);
            kq = wave_sum(kq);
            const float inv = 1.0f / (rt + s);
            const float mr = mu / rt;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                kap[c] = ph[c] * kk[c] * inv;
                p[c] = ph[c] / (1.0f + mr * kk[c] * kk[c] * ph[c]);
            }
            mq = kq * inv;
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) chan[wave][lane + 64 * c] = make_float4(aa[c], kk[c], qq[c], kap[c]);
        wave_lds_sync();

        float A[4] = {0.f, 0.f, 0.f, 0.f}, Bq[4] = {0.f, 0.f, 0.f, 0.f};
        float kr[RPT];
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const float4 c4 = chan[wave][rg + 8 * m];
            kr[m] = c4.w;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                S[m][j] *= c4.x;
                A[j] += S[m][j] * c4.y;
                Bq[j] += S[m][j] * c4.z;
            }
        }
#pragma unroll
        for (int off = 8; off <= 32; off <<= 1) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                A[j] += __shfl_xor(A[j], off, 64);
                Bq[j] += __shfl_xor(Bq[j], off, 64);
            }
        }
        float d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = to_f32(v[tok * DV + col + j]) - A[j];
#pragma unroll
        for (int m = 0; m < RPT; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[m][j] += kr[m] * d[j];
        if (rg == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) from_f32(o + tok * DV + col + j, Bq[j] + mq * d[j]);
        }
        wave_lds_sync();  // chan is rewritten by the next token
    }

#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + 8 * m;
        *reinterpret_cast<float4*>(S_T + sbase + size_t(i) * DV + col) =
            make_float4(S[m][0], S[m][1], S[m][2], S[m][3]);
    }
    if (wave == (GR ? 2 * grp : 0)) {  // the first wave of each group
        if (ISO) {
            if (lane == 0) p_T[unit] = pb;
        } else {
#pragma unroll
            for (int c = 0; c < CPL; ++c) p_T[(size_t(unit) * NG + grp) * DK + lane + 64 * c] = p[c];
        }
    }
}

template <int DK, int DV, int VAR, typename Tin, bool GR = false>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
    const long units = long(a.B) * a.H;
    if (units == 0) return hipSuccess;
    hipLaunchKernelGGL((kdn_recurrent_kernel<DK, DV, VAR, Tin, GR>), dim3(unsigned(units)),
                       dim3(DV * 2), 0, stream, static_cast<const Tin*>(a.q),
                       static_cast<const Tin*>(a.k), static_cast<const Tin*>(a.v),
                       static_cast<const Tin*>(a.alpha), static_cast<const Tin*>(a.omega),
                       static_cast<const Tin*>(a.r), a.c0, a.mu, a.T, a.H, a.S0, a.p0,
                       static_cast<Tin*>(a.o), a.S_T, a.p_T, a.cu_seqlens, a.seq_order, a.B,
                       a.gates ? 1 : 0);
    return hipGetLastError();
}

template <int DK, int DV, int VAR, bool GR = false>
hipError_t launch_dtype(const FwdArgs& a, hipStream_t s) {
    return a.dtype == 1 ? launch_t<DK, DV, VAR, bf16_t, GR>(a, s) : launch_t<DK, DV, VAR, float, GR>(a, s);
}

template <int DK, int DV>
hipError_t launch_variant(const FwdArgs& a, hipStream_t s) {
    if (a.variant == 3) return launch_dtype<DK, DV, 0, true>(a, s);  // grouped observation noise
    if (a.variant == 2) return launch_dtype<DK, DV, 2>(a, s);
    return a.variant == 1 ? launch_dtype<DK, DV, 1>(a, s) : launch_dtype<DK, DV, 0>(a, s);
}

}  // namespace

hipError_t launch_recurrent(const FwdArgs& a, hipStream_t stream) {
    if (a.dk == 128 && a.dv == 128) return launch_variant<128, 128>(a, stream);
    if (a.dk == 128 && a.dv == 64) return launch_variant<128, 64>(a, stream);
    if (a.dk == 64 && a.dv == 128) return launch_variant<64, 128>(a, stream);
    if (a.dk == 64 && a.dv == 64) return launch_variant<64, 64>(a, stream);
    return hipErrorNotSupported;
}

}  // namespace kdn
