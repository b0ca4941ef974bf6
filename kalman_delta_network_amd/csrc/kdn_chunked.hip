// kdn_chunked.hip -- chunkwise forward of the KDN recurrence on gfx950
// matrix cores (MFMA).
//
// The sequence of each (batch, head) pair is cut into chunks of L = 64
// tokens.  The memory S (d_k x d_v, fp32) is carried from chunk to chunk in
// registers; inside a chunk all 64 writes are applied at once.
//
// Derivation (our own, from the per-token recurrence of the KDN summary
// page, method steps 2-5).  Inside a chunk write g_t for the cumulative
// decay prod_{s<=t} alpha_s (per key channel), kappa'_t = p_hat_t * k_t (the
// gain numerator) and d_t = r_t + sum_i p_hat_t,i k_t,i^2 (the gain
// denominator), so kappa_t = kappa'_t / d_t.  With
//   Kt_t = k_t * g_t,   Qt_t = q_t * g_t,   Kh_t = kappa'_t / g_t,
//   Kb_t = kappa'_t * g_L / g_t                (g_L: decay over the chunk)
// the innovations delta_t = v_t - (diag(alpha_t) S_{t-1})^T k_t satisfy,
// for Dn_t = delta_t / d_t,
//   M Dn = V - Kt S_c,   M = diag(r) + tril(Kt Kh^T)   (diagonal included:
//                                                     its diagonal is d_t)
//   O    = Qt S_c + tril(Qt Kh^T) Dn
//   S_{c+1} = diag(g_L) S_c + Kb^T Dn
// which reproduces the token recurrence exactly (up to rounding).  The
// gain denominator therefore never needs a separate reduction: it is the
// diagonal of the same matrix product that couples the tokens.  M is lower
// triangular; it is solved by 16 x 16 blocks: the four diagonal blocks are
// inverted in fp32 (forward substitution), the block substitution runs on
// MFMA.
//
// Work decomposition: one workgroup per (batch, head, 64-column tile of
// d_v); 4 waves.  The per-channel part (uncertainty predict / posterior,
// decay products, MFMA operands) is computed by every tile of a head; the
// column part is split across waves, 16 value columns each.  Operands are
// bf16 with fp32 accumulation; the state and the uncertainty stay fp32.
#include "kdn_internal.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kdn {
namespace {

constexpr int L = 64;     // chunk length
constexpr int NWAVE = 4;  // waves per workgroup
constexpr int DVT = 64;   // value columns per workgroup

typedef uint16_t bf16_t;
typedef short s4 __attribute__((ext_vector_type(4)));
typedef __bf16 b4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float ld_f32(const bf16_t* p, size_t i) {
    return __uint_as_float(uint32_t(p[i]) << 16);
}

__device__ __forceinline__ s4 pack4(f4 x) {
    b4 b;
    b[0] = (__bf16)x[0];
    b[1] = (__bf16)x[1];
    b[2] = (__bf16)x[2];
    b[3] = (__bf16)x[3];
    return __builtin_bit_cast(s4, b);
}

__device__ __forceinline__ s4 lds4(const __bf16* p) { return *reinterpret_cast<const s4*>(p); }

__device__ __forceinline__ f4 mfma16(s4 a, s4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void st_out(bf16_t* p, float x) {
    __bf16 b = (__bf16)x;
    *p = __builtin_bit_cast(bf16_t, b);
}

template <int DK>
struct Smem {
    static constexpr int PK = DK + 8;   // pitch of [L][DK] tiles (bf16)
    static constexpr int PL = L + 8;    // pitch of [*][L] tiles (bf16)
    static constexpr int PV = DVT + 8;  // pitch of the v tile (bf16)
    __bf16 Kn[L * PK];      // -k_t * g_t
    __bf16 Qt[L * PK];      // q_t * g_t
    __bf16 Kh[L * PK];      // kappa'_t / g_t
    __bf16 KbT[DK * PL];    // (kappa'_t * g_L / g_t)^T, [channel][token]
    __bf16 Mn[L * PL];      // -M below the diagonal blocks
    __bf16 QK[L * PL];      // tril(Qt Kh^T)
    __bf16 Td[4 * 16 * 16]; // inverses of M's diagonal 16x16 blocks [block][t][s]
    __bf16 Vt[L * PV];      // v tile of this workgroup's columns
    float Md[4 * 16 * 17];  // M's diagonal blocks, fp32 [block][t][s]
    float cr[L];            // mu / r_t (diagonal) or mu / (d_k r_t) (isotropic)
    float rr[L];            // r_t (1 for padding tokens)
    float nn[L];            // |k_t|^2 (isotropic)
    float bh[L];            // b_hat_t (isotropic)
    float gs[L];            // scalar decay products (isotropic)
    float gL[DK];           // g_L per channel
};

template <int DK, bool ISO>
__global__ void __launch_bounds__(NWAVE * 64)
kdn_chunk_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                 const bf16_t* __restrict__ v, const bf16_t* __restrict__ alpha,
                 const bf16_t* __restrict__ omega, const bf16_t* __restrict__ r,
                 const float* __restrict__ c0, float mu, int T, int H, int DV, int units,
                 const float* S0, const float* __restrict__ p0, bf16_t* __restrict__ o,
                 float* S_T, float* __restrict__ p_T) {
    using SM = Smem<DK>;
    constexpr int PK = SM::PK, PL = SM::PL, PV = SM::PV;
    constexpr int KT = DK / 16;  // 16-row tiles of the key dimension
    __shared__ SM sm;

    // block -> (unit, column tile); the tiles of one unit share an XCD
    const int ntile = DV / DVT;
    const int bid = blockIdx.x;
    const int unit = (bid / (8 * ntile)) * 8 + (bid % 8);
    const int tile = (bid / 8) % ntile;
    if (unit >= units) return;
    const int h = unit % H;
    const size_t b = size_t(unit / H);
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int n = lane & 15;  // MFMA column / A-operand row within a 16-tile
    const int g4 = (lane >> 4) * 4;
    const int col = tile * DVT + wave * 16 + n;  // this lane's value column

    // ---- initial state ----
    f4 S[KT];
    const size_t sbase = size_t(unit) * DK * DV;
#pragma unroll
    for (int it = 0; it < KT; ++it)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[it][e] = S0 ? S0[sbase + size_t(16 * it + g4 + e) * DV + col] : 0.f;
    float p = 0.f;  // diagonal: channel `tid` (tid < DK); isotropic: thread 0
    if (ISO) {
        if (tid == 0) p = p0 ? p0[unit] : c0[h];
    } else if (tid < DK) {
        p = p0 ? p0[size_t(unit) * DK + tid] : c0[h];
    }

    const int nchunks = (T + L - 1) / L;
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * L;
        const int nvalid = min(L, T - t0);
        auto tokidx = [&](int t) { return (b * size_t(T) + size_t(t0 + t)) * size_t(H) + size_t(h); };

        // ---- phase 1: per-token scalars and the v tile ----
        if (tid < L) {
            const int t = tid;
            float rt = 1.f, cc = 0.f, nk = 0.f;
            if (t < nvalid) {
                rt = ld_f32(r, tokidx(t));
                cc = ISO ? mu / (float(DK) * rt) : mu / rt;
                if (ISO) {
                    const bf16_t* kr = k + tokidx(t) * DK;
                    for (int i = 0; i < DK; ++i) {
                        const float x = ld_f32(kr, i);
                        nk += x * x;
                    }
                }
            }
            sm.rr[t] = rt;
            sm.cr[t] = cc;
            sm.nn[t] = nk;
        }
        for (int e = tid; e < L * DVT; e += NWAVE * 64) {
            const int t = e / DVT, j = e % DVT;
            const float x = t < nvalid ? ld_f32(v, tokidx(t) * size_t(DV) + tile * DVT + j) : 0.f;
            sm.Vt[t * PV + j] = (__bf16)x;
        }
        __syncthreads();
        if (ISO && tid == 0) {
            // scalar uncertainty chain of the chunk (trace-projected predict,
            // averaged precision increment)
            float g = 1.f;
            for (int t = 0; t < L; ++t) {
                float a = 1.f, w = 0.f;
                if (t < nvalid) {
                    a = ld_f32(alpha, tokidx(t));
                    w = ld_f32(omega, tokidx(t));
                }
                const float ph = a * a * p + w * (1.f / float(DK));
                p = ph / (1.f + sm.cr[t] * sm.nn[t] * ph);
                g *= a;
                sm.bh[t] = ph;
                sm.gs[t] = g;
            }
        }
        if (ISO) __syncthreads();

        // ---- phase 2: per-channel recurrence and MFMA operands ----
        if (tid < DK) {
            const int i = tid;
            float g = 1.f;
            float kh[L];
#pragma unroll
            for (int t = 0; t < L; ++t) {
                float a = 1.f, w = 0.f, kk = 0.f, qq = 0.f;
                if (t < nvalid) {
                    const size_t base = tokidx(t) * DK + i;
                    kk = ld_f32(k, base);
                    qq = ld_f32(q, base);
                    if (!ISO) {
                        a = ld_f32(alpha, base);
                        w = ld_f32(omega, base);
                    }
                }
                float ph;
                if (ISO) {
                    ph = sm.bh[t];
                    g = sm.gs[t];
                } else {
                    ph = a * a * p + w;
                    p = ph / (1.f + sm.cr[t] * kk * kk * ph);
                    g *= a;
                }
                sm.Kn[t * PK + i] = (__bf16)(-kk * g);
                sm.Qt[t * PK + i] = (__bf16)(qq * g);
                kh[t] = ph * kk / g;
            }
            sm.gL[i] = g;
#pragma unroll
            for (int t = 0; t < L; ++t) {
                sm.Kh[t * PK + i] = (__bf16)kh[t];
                sm.KbT[i * PL + t] = (__bf16)(kh[t] * g);
            }
        }
        __syncthreads();

        // ---- phase 3: M = diag(r) + tril(Kt Kh^T) and tril(Qt Kh^T) ----
        for (int job = wave; job < 20; job += NWAVE) {
            const bool isM = job < 10;
            int jt = isM ? job : job - 10;
            int a = 0;
            while (jt > a) { jt -= a + 1; ++a; }
            const int bb = jt;  // tile (a, bb), bb <= a
            const __bf16* A = isM ? sm.Kn : sm.Qt;
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KT; ++kb)
                acc = mfma16(lds4(A + (16 * a + n) * PK + 16 * kb + g4),
                             lds4(sm.Kh + (16 * bb + n) * PK + 16 * kb + g4), acc);
            // acc[e] holds row t = 16a + g4 + e, column s = 16bb + n
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tl = g4 + e, sl = n;
                const int t = 16 * a + tl, s = 16 * bb + sl;
                if (isM) {
                    if (a == bb) {
                        float mv = 0.f;
                        if (sl < tl) mv = -acc[e];
                        if (sl == tl) mv = sm.rr[t] - acc[e];
                        sm.Md[(a * 16 + tl) * 17 + sl] = mv;
                    } else {
                        sm.Mn[t * PL + s] = (__bf16)acc[e];
                    }
                } else {
                    sm.QK[t * PL + s] = (__bf16)((a != bb || sl <= tl) ? acc[e] : 0.f);
                }
            }
        }
        __syncthreads();

        // ---- phase 4: inverses of M's diagonal blocks (fp32) ----
        if (wave == 0) {
            const int a = lane >> 4, s = lane & 15;
            const float* Mb = sm.Md + a * 16 * 17;
            float X[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float acc = (t == s) ? 1.f : 0.f;
#pragma unroll
                for (int u = 0; u < t; ++u) acc -= Mb[t * 17 + u] * X[u];
                X[t] = acc / Mb[t * 17 + t];
                sm.Td[(a * 16 + t) * 16 + s] = (__bf16)X[t];
            }
        }
        __syncthreads();

        // ---- phase 5: column part (wave = 16 value columns) ----
        f4 Dl[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f4 acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = (float)sm.Vt[(16 * a + g4 + e) * PV + wave * 16 + n];
            // R_a = V_a - Kt_a S_c
#pragma unroll
            for (int kb = 0; kb < KT; ++kb) acc = mfma16(lds4(sm.Kn + (16 * a + n) * PK + 16 * kb + g4), pack4(S[kb]), acc);
            // subtract the coupling to earlier blocks: - M_ab Dn_b
#pragma unroll
            for (int bb = 0; bb < a; ++bb) acc = mfma16(lds4(sm.Mn + (16 * a + n) * PL + 16 * bb + g4), pack4(Dl[bb]), acc);
            const f4 zero = {0.f, 0.f, 0.f, 0.f};
            Dl[a] = mfma16(lds4(sm.Td + (a * 16 + n) * 16 + g4), pack4(acc), zero);
        }
        // O = Qt S_c + tril(Qt Kh^T) Dn
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KT; ++kb) acc = mfma16(lds4(sm.Qt + (16 * a + n) * PK + 16 * kb + g4), pack4(S[kb]), acc);
#pragma unroll
            for (int bb = 0; bb <= a; ++bb) acc = mfma16(lds4(sm.QK + (16 * a + n) * PL + 16 * bb + g4), pack4(Dl[bb]), acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * a + g4 + e;
                if (t < nvalid) st_out(o + tokidx(t) * size_t(DV) + col, acc[e]);
            }
        }
        // S_{c+1} = diag(g_L) S_c + Kb^T Dn
#pragma unroll
        for (int it = 0; it < KT; ++it) {
#pragma unroll
            for (int e = 0; e < 4; ++e) S[it][e] *= sm.gL[16 * it + g4 + e];
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
                S[it] = mfma16(lds4(sm.KbT + (16 * it + n) * PL + 16 * bb + g4), pack4(Dl[bb]), S[it]);
        }
        __syncthreads();
    }

    // ---- final state ----
#pragma unroll
    for (int it = 0; it < KT; ++it)
#pragma unroll
        for (int e = 0; e < 4; ++e) S_T[sbase + size_t(16 * it + g4 + e) * DV + col] = S[it][e];
    if (tile == 0) {
        if (ISO) {
            if (tid == 0) p_T[unit] = p;
        } else if (tid < DK) {
            p_T[size_t(unit) * DK + tid] = p;
        }
    }
}

template <int DK, bool ISO>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
    const int units = a.B * a.H;
    if (units == 0) return hipSuccess;
    const int ntile = a.dv / DVT;
    const int groups = (units + 7) / 8;
    const unsigned grid = unsigned(groups) * 8u * unsigned(ntile);
    hipLaunchKernelGGL((kdn_chunk_kernel<DK, ISO>), dim3(grid), dim3(NWAVE * 64), 0, stream,
                       static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                       static_cast<const bf16_t*>(a.v), static_cast<const bf16_t*>(a.alpha),
                       static_cast<const bf16_t*>(a.omega), static_cast<const bf16_t*>(a.r), a.c0,
                       a.mu, a.T, a.H, a.dv, units, a.S0, a.p0, static_cast<bf16_t*>(a.o), a.S_T,
                       a.p_T);
    return hipGetLastError();
}

}  // namespace

bool chunked_supports(const FwdArgs& a) {
    return a.dtype == 1 && (a.dk == 64 || a.dk == 128) && (a.dv % DVT) == 0 && a.dv >= DVT;
}

hipError_t launch_chunked(const FwdArgs& a, hipStream_t stream) {
    if (!chunked_supports(a)) return hipErrorNotSupported;
    if (a.dk == 128) return a.variant == 1 ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
    return a.variant == 1 ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
}

}  // namespace kdn
