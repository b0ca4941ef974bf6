// kdn_backward_chunk.hip -- the memory adjoint of the diagonal KDN recurrence
// in chunk form, on the matrix cores (gfx950).
//
// The forward token step ("Kalman Delta Networks: Uncertainty-aware
// Associative Memory", summary page, method steps 2-5) is, per 32-token chunk
// in the midpoint frame of the chunked forward (kdn_chunked.hip):
//   rho_t = g_t / g_15 (t <= 15),  rho_t = prod_{16<=u<=t} alpha_u (t >= 16)
//   Kt = k rho,  Qt = q rho,  Kh = kappa' / rho   (kappa' = p_hat k)
//   Sg = diag(g_15) S_c,  M = diag(r) + tril(Kt Kh^T),  R = V - Kt Sg,
//   Dn = M^-1 R,  O = Qt Sg + tril(Qt Kh^T) Dn,
//   S_{c+1} = diag(gb_31) X,  X = Sg + Kh^T Dn.
// Its adjoint, given dO and the cotangent dS of S_{c+1}:
//   dX = diag(gb_31) dS,  d gb_31 = rowsum(dS . X),
//   dDn = tril(Qt Kh^T)^T dO + Kh dX,  dR = M^-T dDn  (= dv),
//   dSg = Qt^T dO + dX - Kt^T dR,  dS_c = diag(g_15) dSg,
//   d g_15 = rowsum(dSg . Sg) / g_15,
//   dM = tril(-dR Dn^T),  dQK = tril(dO Dn^T),
//   dQt = dO Sg^T + dQK Kh,  dKt = -dR Sg^T + dM Kh,
//   dKh = dQK^T Qt + dM^T Kt + Dn dX^T.
// Per token and key channel that gives dq = dQt rho, the gradient of k
// through Kt, of kappa' through Kh and of rho (w = d rho . rho), and
// through the prefix products of alpha the gradient of alpha.  The token
// recurrence's uncertainty adjoint (kdn_backward.hip) takes the gradient of
// the normalised gain kappa = kappa' / d (d = r + k . kappa' = M_tt) and of k
// with kappa held fixed; with dr_t = dM_tt those are
//   d kappa = d (d kappa'_chunk - k dr),  dk_mem = dk_chunk - kappa' dr,
// linear in the tile's partial sums, so every column tile converts its own.
//
// Work mapping: one workgroup per (batch, head, 64 value columns), 8 waves,
// chunks in reverse order.  Each chunk runs as its two 16-token halves: the
// first half's forward gives the state at the midpoint, then the second
// half's adjoint and the first half's (every 16 x 16 block of M and
// tril(Qt Kh^T) is then one tile, and the block solves are single tiles).
// The chunk-start states (in the midpoint frame, rounded to bf16: the
// adjoint's products take them as bf16 operands) and uncertainties come from
// the chunked forward's checkpoint mode; the chain re-runs the chunk's
// uncertainty recurrence from the stored p.  One launch covers a slab of
// chunks (ChunkWs): its per-token sums go to buffers of one slab, and the
// state's cotangent passes to the next launch (the earlier slab) through
// the workspace.  Waves 0 .. d_k/16 - 1 hold 16
// key rows of the state-sized matrices (Sg, dS, X) in MFMA accumulator
// layout.  Matrix operands whose contraction index runs along the stored
// rows are gathered from LDS (4 or 8 two-byte reads per lane).
#include "kdn_device.h"
#include "kdn_gates.h"
#include "kdn_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <type_traits>

namespace kdn {
namespace {

using namespace dev;

constexpr int L = 32;       // chunk
constexpr int HL = 16;      // half chunk
constexpr int TILE = 64;    // value columns per workgroup
constexpr int NTH = 512;    // 8 waves

template <int DK>
struct CSmem {
    bf16_t K[L * DK];   // raw k, q, alpha, omega of the chunk, [t][i] (rows past T repeat the last token)
    bf16_t Q[L * DK];
    bf16_t A[L * DK];
    bf16_t W[L * DK];
    bf16_t V[L * TILE];   // v of the tile's columns [t][col]
    bf16_t dO[L * TILE];  // dO, [t][col] swizzled
    float rho[L * DK];    // rho_t,i (midpoint frame)
    float kap[L * DK];    // kappa'_t,i; after the half's products w_t,i = d rho . rho
    bf16_t Kt[L * DK];    // [t][i] swizzled
    bf16_t Qt[L * DK];
    bf16_t Kh[L * DK];
    bf16_t S[DK * TILE];   // the half's start state, bf16 [i][col] swizzled
    bf16_t dX[TILE * DK];  // dX of the half, bf16 [col][i] swizzled
    bf16_t R[HL * TILE];   // [t][col] swizzled
    bf16_t Dn[2][HL * TILE];
    bf16_t dDn[HL * TILE];
    bf16_t dR[HL * TILE];
    bf16_t dOT[TILE * L];  // dO transposed, [col][t] swizzled
    bf16_t dRT[TILE * HL]; // dR transposed, [col][t] swizzled
    float Md[2 * 256];     // M's diagonal blocks, column-major [a][s][t]
    float Wi[2][2][64];    // block-inverse scratch
    bf16_t Td[2 * 256];    // their inverses [a][t][s]
    bf16_t QK[2 * 256];    // tril(Qt Kh^T) of each half [a][t][s]
    bf16_t dM[256];        // tril(-dR Dn^T) of the current half [t][s]
    bf16_t dQK[256];       // tril(dO Dn^T) [t][s]
    float r[L];
    float cr[L];           // mu / r_t
    float d[L];            // M_tt = r_t + k_t . kappa'_t
    float dr[L];           // dM_tt
    float GA[DK], GB[DK];  // g_15 and gb_31
    float dGA[DK], dGB[DK];
    float spart[L][DK / 64];  // sum_i p_hat k^2 over each wave's 64 channels (fp32)
    float nk[L][DK / 64];     // gated: |k_t|^2 and |q_t|^2 over each wave's 64 channels
    float nq[L][DK / 64];
    float skv[L], sqv[L];     // gated: 1 / |k_t| and 1 / |q_t|
    float uacc[DK / 16][L];   // sum_i d kappa kappa' over each key tile's 16 channels
};

// The lane index as a value the compiler cannot hoist out of the chunk loop:
// otherwise it keeps every loop-invariant LDS address of the operand reads
// below in registers across the loop (hundreds of them) and spills.
__device__ __forceinline__ int lane_id() {
    int l;
    asm volatile("v_and_b32 %0, 63, %1" : "=v"(l) : "v"(int(threadIdx.x)));
    return l;
}

// ---------------------------------------------------------------------------
// MFMA operands from LDS.  Row operands: lane l reads row row0 + l % 16 of a
// [rows][W] tile at contraction index k0 + 8 (l / 16) (16x16x32) or
// k0 + 4 (l / 16) (16x16x16).  Gathered operands: the contraction index runs
// along the stored rows: lane l reads rows k0 + 8 (l / 16) + j (or 4 (l / 16)
// + j) of column c0 + l % 16.
// ---------------------------------------------------------------------------
template <int W>
__device__ __forceinline__ b8 row32(const bf16_t* A, int row0, int k0) {
    const int lane = lane_id();
    return *reinterpret_cast<const b8*>(A + sw<W>(row0 + (lane & 15), k0 + 8 * (lane >> 4)));
}
template <int W>
__device__ __forceinline__ s4 row16(const bf16_t* A, int row0, int k0) {
    const int lane = lane_id();
    return *reinterpret_cast<const s4*>(A + sw<W>(row0 + (lane & 15), k0 + 4 * (lane >> 4)));
}
template <int W>
__device__ __forceinline__ s4 col16(const bf16_t* A, int k0, int c0) {
    const int lane = lane_id();
    s4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = short(A[sw<W>(k0 + 4 * (lane >> 4) + j, c0 + (lane & 15))]);
    return v;
}
template <int W>
__device__ __forceinline__ b8 col32(const bf16_t* A, int k0, int c0) {
    const int lane = lane_id();
    u4 u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t lo = A[sw<W>(k0 + 8 * (lane >> 4) + 2 * j, c0 + (lane & 15))];
        const uint32_t hi = A[sw<W>(k0 + 8 * (lane >> 4) + 2 * j + 1, c0 + (lane & 15))];
        u[j] = lo | (hi << 16);
    }
    return __builtin_bit_cast(b8, u);
}
// plain 16 x 16 tiles [row][col]
__device__ __forceinline__ s4 row16p(const bf16_t* A) {
    const int lane = lane_id();
    return *reinterpret_cast<const s4*>(A + (lane & 15) * 16 + 4 * (lane >> 4));
}
__device__ __forceinline__ s4 col16p(const bf16_t* A) {
    const int lane = lane_id();
    s4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = short(A[(4 * (lane >> 4) + j) * 16 + (lane & 15)]);
    return v;
}
// accumulator tile (rows row0 + 4 (l / 16) + e, column c0 + l % 16) to a
// swizzled [rows][W] bf16 tile
template <int W>
__device__ __forceinline__ void put(bf16_t* D, int row0, int c0, f4 c) {
    const int lane = lane_id();
#pragma unroll
    for (int e = 0; e < 4; ++e) D[sw<W>(row0 + 4 * (lane >> 4) + e, c0 + (lane & 15))] = to_bf(c[e]);
}

// accumulator tile (rows row0 + 4 (l / 16) + e, column c0 + l % 16) to the
// transposed swizzled [cols][W] tile: the lane's four rows are consecutive
// there (one 8-byte store)
template <int W>
__device__ __forceinline__ void putT(bf16_t* D, int row0, int c0, f4 c) {
    const int lane = lane_id();
    *reinterpret_cast<s4*>(D + sw<W>(c0 + (lane & 15), row0 + 4 * (lane >> 4))) = __builtin_bit_cast(s4, u2{pack2(c[0], c[1]), pack2(c[2], c[3])});
}

constexpr f4 kZero = {0.f, 0.f, 0.f, 0.f};

// One chunk's inputs as each thread loads them, one chunk ahead: its 16-byte
// piece of the raw k, q, alpha, omega tiles and of the v and dO tiles, r
// (threads < 32) and (state waves) its 16 entries of the checkpoint Sg
// (bf16, four rows of a column in each u2).
struct Pre {
    u4 kqaw[4];
    u4 v, d;
    bf16_t r;
    u2 sg[4];
};

__device__ __forceinline__ f4 unpack4(u2 x) {
    return f4{__uint_as_float(x[0] << 16), __uint_as_float(x[0] & 0xffff0000u), __uint_as_float(x[1] << 16),
              __uint_as_float(x[1] & 0xffff0000u)};
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
// GATE: the gated layer's values from raw inputs, as the gated forward forms
// them (alpha = sigmoid(z), omega = softplus(z), r = r_min + softplus(z), q
// and k divided by their norms over the d_k channels)
template <int DK, bool GATE>
__global__ void __launch_bounds__(NTH) kdn_backward_chunk_kernel(BwdArgs A, ChunkWs W, int c_lo, int c_hi) {
    constexpr int NT = DK / 16;     // 16-row tiles of the key dimension (state waves)
    constexpr int NCW = DK / 64;    // chain waves
    __shared__ CSmem<DK> sm;
    const int nunit = A.B * A.H;
    const int ntile = A.dv / TILE;
    const int tile = int(blockIdx.x) / nunit;
    const int unit = int(blockIdx.x) % nunit;
    if (W.flag[unit]) return;  // the recurrent memory adjoint takes this pair
    const int h = unit % A.H;
    const size_t b = size_t(unit / A.H);
    const int T = A.T;
    const int DV = A.dv;
    const int nchunks = (T + L - 1) / L;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = 4 * (lane >> 4);
    const float mu = A.mu;
    const bf16_t* qin = static_cast<const bf16_t*>(A.q);
    const bf16_t* kin = static_cast<const bf16_t*>(A.k);
    const bf16_t* vin = static_cast<const bf16_t*>(A.v);
    const bf16_t* ain = static_cast<const bf16_t*>(A.alpha);
    const bf16_t* win = static_cast<const bf16_t*>(A.omega);
    const bf16_t* rin = static_cast<const bf16_t*>(A.r);
    const bf16_t* doin = static_cast<const bf16_t*>(A.dO);
    const bf16_t* ck = W.cks + (size_t(unit) * ntile + tile) * nchunks * DK * TILE;  // [chunk][DK / 4][64][4]
    const float* ckp = W.ckp + size_t(unit) * nchunks * DK;                          // [chunk][DK]
    const int tb = c_lo * L;  // the slab's first token
    // the slab's per-token buffers, token t at row t - tb: [unit][slab][ntile][4][DK], [unit][slab][DK]
    float* partial = W.partial + size_t(unit) * W.slab * ntile * 4 * DK;
    float* pbuf = W.pbuf + size_t(unit) * W.slab * DK;
    float* tsc = W.tsc + size_t(unit) * T * 8;  // [T][8] per-token sums
    const auto tokidx = [&](int t) { return (b * size_t(T) + size_t(t)) * size_t(A.H) + size_t(h); };

    // the upper 8 x 8 corner of each inverse block is zero (block_inverse
    // writes the rest)
    for (int e = threadIdx.x; e < 2 * 64; e += NTH) sm.Td[(e >> 6) * 256 + ((e >> 3) & 7) * 16 + 8 + (e & 7)] = 0;

    // the cotangent of the state, key rows 16 wave + 4 (l / 16) + e, columns 16
    // ct + l % 16: dS_T at the last slab, else what the later slab left
    const bool stw = wave < NT;
    const float* dsi = c_hi == nchunks ? A.dS_T : W.dsc;
    f4 dS[4], Sg[4], Sm[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        dS[ct] = kZero;
        if (stw && dsi)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dS[ct][e] = dsi[(size_t(unit) * DK + 16 * wave + g4 + e) * DV + tile * TILE + 16 * ct + n];
    }

    Pre pre;
    // chunk c's inputs into pre (rows past T repeat the last token; v and dO
    // rows past T read as zero)
    const auto load = [&](int c) {
        const int tid = threadIdx.x;
        const int t0 = c * L, nvalid = min(L, T - t0), last = nvalid - 1;
        constexpr int PR = DK / 8;
        if (tid < L * PR) {
            const int t = tid / PR, cc = tid % PR;
            const size_t src = tokidx(t0 + min(t, last)) * DK + 8 * cc;
            pre.kqaw[0] = *reinterpret_cast<const u4*>(kin + src);
            pre.kqaw[1] = *reinterpret_cast<const u4*>(qin + src);
            pre.kqaw[2] = *reinterpret_cast<const u4*>(ain + src);
            pre.kqaw[3] = *reinterpret_cast<const u4*>(win + src);
        }
        if (tid < L * 8) {
            const int t = tid / 8, cc = tid % 8;
            const bool ok = t < nvalid;
            const size_t src = tokidx(t0 + min(t, last)) * DV + tile * TILE + 8 * cc;
            const u4 zero = {0u, 0u, 0u, 0u};
            pre.v = ok ? *reinterpret_cast<const u4*>(vin + src) : zero;
            pre.d = (ok && doin) ? *reinterpret_cast<const u4*>(doin + src) : zero;
        }
        if (tid < L) pre.r = rin[tokidx(t0 + min(tid, last))];
        if (stw) {
            // [DK / 4][64][4]: rows 4 (l / 16) .. + 3 of the wave's 16 in one load
            const u2* ckc = reinterpret_cast<const u2*>(ck + size_t(c) * DK * TILE);
            const int ln = threadIdx.x & 63;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) pre.sg[ct] = ckc[(4 * wave + (ln >> 4)) * TILE + 16 * ct + (ln & 15)];
        }
    };
    load(c_hi - 1);
    for (int c = c_hi - 1; c >= c_lo; --c) {
        const int lane = lane_id();  // (see lane_id)
        const int n = lane & 15, g4 = 4 * (lane >> 4);
        const int t0 = c * L;
        const int nvalid = min(L, T - t0);
        // ---- this chunk's inputs (loaded one chunk ahead) into LDS ----
        {
            const int tid = threadIdx.x;
            constexpr int PR = DK / 8;  // 16-byte pieces per row
            if (tid < L * PR) {
                const int t = tid / PR, cc = tid % PR;
                *reinterpret_cast<u4*>(&sm.K[t * DK + 8 * cc]) = pre.kqaw[0];
                *reinterpret_cast<u4*>(&sm.Q[t * DK + 8 * cc]) = pre.kqaw[1];
                *reinterpret_cast<u4*>(&sm.A[t * DK + 8 * cc]) = pre.kqaw[2];
                *reinterpret_cast<u4*>(&sm.W[t * DK + 8 * cc]) = pre.kqaw[3];
            }
            if (tid < L * 8) {
                const int t = tid / 8, cc = tid % 8;
                *reinterpret_cast<u4*>(&sm.V[t * TILE + 8 * cc]) = pre.v;
                *reinterpret_cast<u4*>(&sm.dO[sw<TILE>(t, 8 * cc)]) = pre.d;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sm.dOT[sw<L>(8 * cc + 2 * j, t)] = bf16_t(pre.d[j] & 0xffffu);
                    sm.dOT[sw<L>(8 * cc + 2 * j + 1, t)] = bf16_t(pre.d[j] >> 16);
                }
            }
            if (tid < L) {
                float rz = bf1(pre.r);
                if (GATE) rz = kGateRMin + gate_softplus(rz);
                const float rt = tid < nvalid ? rz : 1.f;
                sm.r[tid] = rt;
                sm.cr[tid] = mu / rt;
            }
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) Sg[ct] = unpack4(pre.sg[ct]);
        }
        bar();
        if (c > c_lo) load(c - 1);  // the next chunk's inputs, in flight during this one
        if constexpr (GATE) {
            // |k_t|^2 and |q_t|^2, a wave covering 64 channels of one token per step
#pragma unroll 1
            for (int j = 0; j < L * DK / NTH; ++j) {
                const int e = threadIdx.x + NTH * j;
                const int t = e / DK, i = e % DK;
                const float xk = bf1(sm.K[e]), xq = bf1(sm.Q[e]);
                float a = xk * xk, b2 = xq * xq;
                a = sum16(a);
                a = halve16(a, a);
                a = halve32(a, a);
                b2 = sum16(b2);
                b2 = halve16(b2, b2);
                b2 = halve32(b2, b2);
                if (lane == 0) {
                    sm.nk[t][i / 64] = a;
                    sm.nq[t][i / 64] = b2;
                }
            }
            bar();
        }
        // gated: the prologue's 1 / |k_t| and 1 / |q_t|; otherwise 1
        const auto kscale = [&](int t) {
            if constexpr (!GATE) return 1.f;
            float a = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < DK / 64; ++w2) a += sm.nk[t][w2];
            return inv_norm(a);
        };
        const auto qscale = [&](int t) {
            if constexpr (!GATE) return 1.f;
            float a = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < DK / 64; ++w2) a += sm.nq[t][w2];
            return inv_norm(a);
        };
        // ---- chain: uncertainty recurrence, decays, the chunk's operands ----
        // (MASK: a tail chunk; padding tokens take alpha = 1, k = q = omega = 0)
        const auto chain = [&](auto maskc) {
            constexpr bool MASK = decltype(maskc)::value;
            const int i = 64 * wave + lane;
            // the first half's 1 / rho_t = prod_{t<u<=15} alpha_u, from the
            // midpoint backwards (registers)
            float hr[HL], a0;
            {
                float a16[HL];
#pragma unroll
                for (int t = 0; t < HL; ++t) {
                    float x = bf1(sm.A[t * DK + i]);
                    if (GATE) x = gate_sigmoid(x);
                    a16[t] = (!MASK || t < nvalid) ? x : 1.f;
                }
                hr[HL - 1] = 1.f;
#pragma unroll
                for (int t = HL - 2; t >= 0; --t) hr[t] = hr[t + 1] * a16[t + 1];
                a0 = a16[0];
            }
            const float ga = hr[0] * a0;  // g_15
            float p = ckp[size_t(c) * DK + i];
            float gb = 1.f;
            // eight tokens at a time: every LDS read of a group is issued
            // before its recurrence starts.  The chain keeps to the
            // sequential part (p_hat and rho per token); every wave forms the
            // operands from them below.
#pragma unroll
            for (int b8i = 0; b8i < L / 8; ++b8i) {
                float al[8], kk[8], w[8], cv[8], pv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int t = 8 * b8i + j;
                    const bool ok = !MASK || t < nvalid;
                    float xa = bf1(sm.A[t * DK + i]), xk = bf1(sm.K[t * DK + i]);
                    float xw = bf1(sm.W[t * DK + i]);
                    if (GATE) {
                        xa = gate_sigmoid(xa);
                        xw = gate_softplus(xw);
                        xk *= kscale(t);
                    }
                    al[j] = ok ? xa : 1.f;
                    kk[j] = ok ? xk : 0.f;
                    w[j] = ok ? xw : 0.f;
                    cv[j] = sm.cr[t];
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int t = 8 * b8i + j;
                    pv[j] = p;
                    const float ph = fmaf(al[j] * al[j], p, w[j]);
                    // the forward chain's arithmetic: p' = p_hat / (1 + (mu / r) k^2 p_hat)
                    p = ph * __builtin_amdgcn_rcpf(fmaf(cv[j] * kk[j], ph * kk[j], 1.f));
                    float rh;
                    if (t < HL) {
                        rh = __builtin_amdgcn_rcpf(hr[t]);
                    } else {
                        gb *= al[j];
                        rh = gb;
                    }
                    sm.rho[t * DK + i] = rh;
                    sm.kap[t * DK + i] = ph;  // p_hat until the operands are formed
                }
                if (tile == 0)  // p_{t-1} of the group's tokens
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int t = 8 * b8i + j;
                        if (!MASK || t < nvalid) __builtin_nontemporal_store(pv[j], &pbuf[size_t(t0 - tb + t) * DK + i]);
                    }
                asm volatile("" ::: "memory");  // one group at a time
            }
            sm.GA[i] = ga;
            sm.GB[i] = gb;
        };
        if (wave < NCW) {
            if (nvalid == L) chain(std::false_type{});
            else chain(std::true_type{});
        } else if (GATE && wave == NCW && lane < L) {
            sm.skv[lane] = kscale(lane);
            sm.sqv[lane] = qscale(lane);
        }
        bar();
        // the chunk's operands from p_hat and rho (every wave): kappa' =
        // p_hat k, Kt = k rho, Qt = q rho, Kh = kappa' / rho; and the gain
        // denominators' sums p_hat k^2 in fp32 (a wave covers 64 channels of
        // one token per step)
#pragma unroll
        for (int j = 0; j < L * DK / NTH; ++j) {
            const int e = threadIdx.x + NTH * j;
            const int t = e / DK, i = e % DK;
            const bool ok = t < nvalid;
            const float xk = bf1(sm.K[e]) * (GATE ? sm.skv[t] : 1.f), xq = bf1(sm.Q[e]) * (GATE ? sm.sqv[t] : 1.f);
            const float kk = ok ? xk : 0.f, qq = ok ? xq : 0.f;
            const float rh = sm.rho[e];
            const float kap = sm.kap[e] * kk;
            sm.kap[e] = kap;
            sm.Kt[sw<DK>(t, i)] = to_bf(kk * rh);
            sm.Qt[sw<DK>(t, i)] = to_bf(qq * rh);
            sm.Kh[sw<DK>(t, i)] = to_bf(kap * __builtin_amdgcn_rcpf(rh));
            float sk = sum16(kap * kk);
            sk = halve16(sk, sk);
            sk = halve32(sk, sk);
            if (lane == 0) sm.spart[t][i / 64] = sk;
        }
        if (stw) {
            // the first half's start state as bf16
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) put<TILE>(sm.S, 16 * wave, 16 * ct, Sg[ct]);
        }
        bar();
        // ---- M's diagonal blocks and tril(Qt Kh^T) of both halves ----
        if (wave < 4) {
            const int a = wave & 1;
            const bf16_t* X = wave < 2 ? sm.Kt : sm.Qt;
            f4 acc = kZero;
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += 32) acc = mfma32(row32<DK>(X, HL * a, k0), row32<DK>(sm.Kh, HL * a, k0), acc);
            // acc[e] = row t = g4 + e, column s = n
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = g4 + e;
                if (wave < 2) {
                    const float m = t > n ? acc[e] : t == n ? acc[e] + sm.r[HL * a + t] : 0.f;
                    sm.Md[a * 256 + n * 16 + t] = m;
                    if (t == n) sm.d[HL * a + t] = m;
                } else {
                    sm.QK[a * 256 + t * 16 + n] = to_bf(t >= n ? acc[e] : 0.f);
                }
            }
        }
        bar();
        if (wave == 0) block_inverse(sm.Md, sm.Wi, sm.Td, lane);
        // R of the first half: V - Kt Sg (waves 4..7, one 16-column tile each)
        if (wave >= 4) {
            const int ct = wave - 4;
            f4 acc = kZero;
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += 32) acc = mfma32(row32<DK>(sm.Kt, 0, k0), col32<TILE>(sm.S, k0, 16 * ct), acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = bf1(sm.V[(g4 + e) * TILE + 16 * ct + n]) - acc[e];
            put<TILE>(sm.R, 0, 16 * ct, acc);
        }
        bar();
        // Dn of the first half: T_A R
        if (wave < 4) {
            const int ct = wave;
            const f4 acc = mfma16(row16p(sm.Td), col16<TILE>(sm.R, 0, 16 * ct), kZero);
            put<TILE>(sm.Dn[0], 0, 16 * ct, acc);
        }
        bar();
        // the midpoint state Sm = Sg + Kh_A^T Dn_A (state waves), as bf16 for
        // the second half
        if (stw) {
            const s4 ak = col16<DK>(sm.Kh, 0, 16 * wave);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                Sm[ct] = mfma16(ak, col16<TILE>(sm.Dn[0], 0, 16 * ct), Sg[ct]);
                put<TILE>(sm.S, 16 * wave, 16 * ct, Sm[ct]);
            }
        }
        bar();
        // R of the second half: V - Kt Sm
        if (wave >= 4) {
            const int ct = wave - 4;
            f4 acc = kZero;
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += 32) acc = mfma32(row32<DK>(sm.Kt, HL, k0), col32<TILE>(sm.S, k0, 16 * ct), acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = bf1(sm.V[(HL + g4 + e) * TILE + 16 * ct + n]) - acc[e];
            put<TILE>(sm.R, 0, 16 * ct, acc);
        }
        bar();
        if (wave < 4) {
            const int ct = wave;
            const f4 acc = mfma16(row16p(sm.Td + 256), col16<TILE>(sm.R, 0, 16 * ct), kZero);
            put<TILE>(sm.Dn[1], 0, 16 * ct, acc);
        }
        bar();
        // X = Sm + Kh_B^T Dn_B, d gb_31 = rowsum(dS . X), dX = diag(gb_31) dS
        if (stw) {
            const s4 ak = col16<DK>(sm.Kh, HL, 16 * wave);
            f4 part = kZero;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const f4 x = mfma16(ak, col16<TILE>(sm.Dn[1], 0, 16 * ct), Sm[ct]);
                part += dS[ct] * x;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float s = sum16(part[e]);
                const int i = 16 * wave + g4 + e;
                if (n == 0) sm.dGB[i] = s;
                const float gbi = sm.GB[i];
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) dS[ct][e] *= gbi;  // dS now holds dX
            }
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) putT<DK>(sm.dX, 16 * wave, 16 * ct, dS[ct]);
        }
        bar();

        // ---- the adjoint of each half, the second first ----
#pragma unroll 1
        for (int half = 1; half >= 0; --half) {
            const int th = HL * half;
            const bf16_t* Tinv = sm.Td + 256 * half;
            const bf16_t* QKh = sm.QK + 256 * half;
            const bf16_t* Dnh = sm.Dn[half];
            // dDn = QK^T dO + Kh dX
            if (wave < 4) {
                const int ct = wave;
                f4 acc = mfma16(col16p(QKh), row16<L>(sm.dOT, 16 * ct, th), kZero);
#pragma unroll
                for (int k0 = 0; k0 < DK; k0 += 32) acc = mfma32(row32<DK>(sm.Kh, th, k0), row32<DK>(sm.dX, 16 * ct, k0), acc);
                put<TILE>(sm.dDn, 0, 16 * ct, acc);
            }
            bar();
            // dR = T^T dDn (= dv)
            if (wave < 4) {
                const int ct = wave;
                const f4 acc = mfma16(col16p(Tinv), col16<TILE>(sm.dDn, 0, 16 * ct), kZero);
                put<TILE>(sm.dR, 0, 16 * ct, acc);
                putT<HL>(sm.dRT, 0, 16 * ct, acc);
                if (A.dv_)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = th + g4 + e;
                        if (t < nvalid) A.dv_[tokidx(t0 + t) * DV + tile * TILE + 16 * ct + n] = acc[e];
                    }
            }
            bar();
            if (stw) {
                // dS_start = dX + Qt^T dO - Kt^T dR
                const s4 aq = col16<DK>(sm.Qt, th, 16 * wave), akt = col16<DK>(sm.Kt, th, 16 * wave);
                f4 part = kZero;
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const f4 pos = mfma16(aq, row16<L>(sm.dOT, 16 * ct, th), dS[ct]);
                    const f4 neg = mfma16(akt, row16<HL>(sm.dRT, 16 * ct, 0), kZero);
                    dS[ct] = pos - neg;
                    if (half == 0) part += dS[ct] * Sg[ct];
                }
                if (half == 0) {
                    // d g_15 = rowsum(dSg . Sg) / g_15; the previous chunk's dS = diag(g_15) dSg
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float s = sum16(part[e]);
                        const int i = 16 * wave + g4 + e;
                        const float ga = sm.GA[i];
                        if (n == 0) sm.dGA[i] = s / ga;
#pragma unroll
                        for (int ct = 0; ct < 4; ++ct) dS[ct][e] *= ga;
                    }
                }
            }
            // dM = tril(-dR Dn^T) and dQK = tril(dO Dn^T) on two waves (after
            // their state work at d_k = 128, where every wave is a state wave)
            constexpr int WM = NT < 6 ? NT : 6;
            if (wave == WM || wave == WM + 1) {
                const bool isM = wave == WM;
                f4 acc = kZero;
#pragma unroll
                for (int k0 = 0; k0 < TILE; k0 += 32)
                    acc = mfma32(isM ? row32<TILE>(sm.dR, 0, k0) : row32<TILE>(sm.dO, th, k0), row32<TILE>(Dnh, 0, k0), acc);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = g4 + e;
                    if (isM) {
                        sm.dM[t * 16 + n] = to_bf(t >= n ? -acc[e] : 0.f);
                        if (t == n) sm.dr[th + t] = -acc[e];
                    } else {
                        sm.dQK[t * 16 + n] = to_bf(t >= n ? acc[e] : 0.f);
                    }
                }
            }
            bar();
            // per token and key channel: dQt, dKt, dKh of key tile wave
            if (wave < NT) {
                const int i0 = 16 * wave;
                const bf16_t* Sh = sm.S;  // this half's start state (bf16 [i][col])
                f4 dqt = mfma16(row16p(sm.dQK), col16<DK>(sm.Kh, th, i0), kZero);
                f4 dkt = mfma16(row16p(sm.dM), col16<DK>(sm.Kh, th, i0), kZero);
                f4 dkh = mfma16(col16p(sm.dQK), col16<DK>(sm.Qt, th, i0), kZero);
                dkh = mfma16(col16p(sm.dM), col16<DK>(sm.Kt, th, i0), dkh);
                f4 neg = kZero;
#pragma unroll
                for (int k0 = 0; k0 < TILE; k0 += 32) {
                    const b8 sv = row32<TILE>(Sh, i0, k0);
                    dqt = mfma32(row32<TILE>(sm.dO, th, k0), sv, dqt);
                    neg = mfma32(row32<TILE>(sm.dR, 0, k0), sv, neg);
                    dkh = mfma32(row32<TILE>(Dnh, 0, k0), col32<DK>(sm.dX, k0, i0), dkh);
                }
                dkt -= neg;
                // acc[e]: token th + g4 + e, channel i0 + n
                const int i = i0 + n;
                float uv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tl = th + g4 + e;
                    const float rh = sm.rho[tl * DK + i], kp = sm.kap[tl * DK + i];
                    const float kk = bf1(sm.K[tl * DK + i]) * (GATE ? sm.skv[tl] : 1.f);
                    const float qq = bf1(sm.Q[tl * DK + i]) * (GATE ? sm.sqv[tl] : 1.f);
                    const float dq = dqt[e] * rh, dkc = dkt[e] * rh, dkapc = dkh[e] * __builtin_amdgcn_rcpf(rh);
                    const float drt = sm.dr[tl], dt = sm.d[tl];
                    const float dkap = dt * fmaf(-kk, drt, dkapc);
                    uv[e] = dkap * kp;
                    sm.kap[tl * DK + i] = fmaf(dkc, kk, fmaf(dq, qq, -dkapc * kp));  // w = d rho . rho
                    if (tl < nvalid) {
                        float* dst = partial + (size_t(t0 - tb + tl) * ntile + tile) * 4 * DK + i;
                        __builtin_nontemporal_store(dq, &dst[0]);
                        __builtin_nontemporal_store(dkap, &dst[DK]);
                        __builtin_nontemporal_store(fmaf(-kp, drt, dkc), &dst[2 * DK]);
                    }
                }
                // u_t = sum_i d kappa kappa' over the key tile's 16 channels
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float su = sum16(uv[e]);
                    if (n == 0) sm.uacc[wave][th + g4 + e] = su;
                }
            }
            bar();
            if (wave == NT - 1 && lane < HL && th + lane < nvalid) {
                // the uncertainty adjoint's per-token sums: u_t of this tile
                // at [tile]; tile 0 also d_t = r_t + sum_i p_hat k^2 at [2]
                // and (gated) 1 / |k_t| at [6]
                float u = 0.f;
#pragma unroll
                for (int w2 = 0; w2 < NT; ++w2) u += sm.uacc[w2][th + lane];
                float* ts = tsc + size_t(t0 + th + lane) * 8;
                ts[tile] = u;
                if (tile == 0) {
                    float sk = sm.r[th + lane];
#pragma unroll
                    for (int w2 = 0; w2 < DK / 64; ++w2) sk += sm.spart[th + lane][w2];
                    ts[2] = sk;
                    if (GATE) ts[6] = sm.skv[th + lane];
                }
            }
            if (half == 1) {
                // the first half: its start state and dX = dS (the state waves
                // hold the cotangent of the midpoint state)
                if (stw)
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct) {
                        put<TILE>(sm.S, 16 * wave, 16 * ct, Sg[ct]);
                        putT<DK>(sm.dX, 16 * wave, 16 * ct, dS[ct]);
                    }
                bar();
            }
        }
        // ---- d alpha of the memory part, per channel over the chunk ----
        const auto scan = [&](auto maskc) {
            constexpr bool MASK = decltype(maskc)::value;
            const int i = 64 * wave + lane;
            const float fa = sm.dGA[i] * sm.GA[i], fb = sm.dGB[i] * sm.GB[i];
            float* dst = partial + (size_t(t0 - tb) * ntile + tile) * 4 * DK + 3 * DK + i;
            const size_t tstep = size_t(ntile) * 4 * DK;
            // u <= 15: -sum_{t<u} w_t + fa;  u >= 16: sum_{t>=u} w_t + fb
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                float wv[HL], av[HL];
#pragma unroll
                for (int j = 0; j < HL; ++j) {
                    const int u = HL * hf + j;
                    wv[j] = sm.kap[u * DK + i];
                    float x = bf1(sm.A[u * DK + i]);
                    if (GATE) x = gate_sigmoid(x);
                    av[j] = (!MASK || u < nvalid) ? x : 1.f;
                }
                float acc = 0.f;
                if (hf == 0) {
#pragma unroll
                    for (int j = 0; j < HL; ++j) {
                        if (!MASK || j < nvalid) __builtin_nontemporal_store((fa - acc) * __builtin_amdgcn_rcpf(av[j]), &dst[j * tstep]);
                        acc += wv[j];
                    }
                } else {
#pragma unroll
                    for (int j = HL - 1; j >= 0; --j) {
                        acc += wv[j];
                        if (!MASK || HL + j < nvalid) __builtin_nontemporal_store((acc + fb) * __builtin_amdgcn_rcpf(av[j]), &dst[(HL + j) * tstep]);
                    }
                }
                asm volatile("" ::: "memory");
            }
        };
        if (wave < NCW) {
            if (nvalid == L) scan(std::false_type{});
            else scan(std::true_type{});
        }
        bar();
    }
    // dS0 after the first slab, else the cotangent the earlier slab starts from
    // (each workgroup reads its own part of it at its start, then writes it)
    float* dso = c_lo == 0 ? A.dS0 : W.dsc;
    if (stw && dso)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dso[(size_t(unit) * DK + 16 * wave + g4 + e) * DV + tile * TILE + 16 * ct + n] = dS[ct][e];
}

// ---------------------------------------------------------------------------
// The uncertainty adjoint after the chunked memory adjoint: one wave per
// (batch, head, 64 key channels), lane = channel, backwards over the tokens.
// The step is the token recurrence's (kdn_backward.hip): with
// p_hat = alpha^2 p_{t-1} + omega, d = r + sum_i p_hat k^2 and
// u = sum_i d kappa p_hat k, the gain's derivatives d kappa / d p_hat = k / d
// and d kappa / dk = p_hat / d and the denominator's dd = -u / d^2, the
// posterior p' = p_hat / (1 + (mu / r) k^2 p_hat); the carried dp and the
// gradients of k, alpha, omega follow per channel.  d and u are sums over
// every channel (and u over the column tiles) that do not depend on dp: the
// chunked kernel leaves them per token in the per-token sums, so the
// channels split over waves with no exchange per token.  dr, a channel sum
// that does depend on dp, is left there per wave and added by
// kdn_backward_dr_kernel.
// The carried dp is affine in itself per token, dp_{t-1} = f_t dp_t + g_t
// with f_t = alpha^2 / den^2 and g_t = alpha^2 (gk k / d + dd k^2), so the
// sequence is cut into segments of SEGU tokens run in parallel: a first
// launch (MAPS) composes each segment's affine map, a second runs every
// segment from its entering dp (the later segments' maps applied in order to
// dp_T) and writes the gradients.  A slab's launches cover its segments; the
// dp a slab leaves for the next is its first segment's map applied to that
// segment's entering dp, so every segment's entering dp is the same chain of
// operations whatever the slab length.  GATE:
// alpha, omega and r are formed from the pre-activations as the gated
// forward forms them, and the written d alpha, d omega (and dr, in
// kdn_backward_dr_kernel) are already the gradients of the pre-activations.
// Per-token sums [t][8]: u of tiles 0 and 1, d, dd, dr of channel halves 0
// and 1, (gated) 1 / |k_t|.
// The per-token tile sums and p_{t-1} (hundreds of MB per slab at B=8,
// H=16, d=128) are written by the memory adjoint and read here with
// nontemporal hints, as are the gradients written here.
// ---------------------------------------------------------------------------
constexpr int PFU = 8;    // prefetch ring: token inputs are loaded 7 tokens ahead
constexpr int SEGU = 64;  // tokens per segment of the uncertainty adjoint (slabs are multiples of it)

struct UncTok {
    float q[2], k[2], ks[2], a[2];  // the tiles' (at most 2) partial sums
    float u[2];
    float d, pp, sk;  // sk (gated): 1 / |k_t|
    bf16_t al, kk, w, r;
};

template <int DK, bool MAPS, bool GATE>
__global__ void __launch_bounds__(64) kdn_backward_unc_chunk_kernel(BwdArgs A, ChunkWs W, int slab, int tb, int te,
                                                                   int nseg) {
    constexpr int NWV = DK / 64;
    const int nunit = A.B * A.H;
    const int ntile = A.dv / TILE;  // 1 or 2
    const int unit = int(blockIdx.x) % nunit;
    const int wv = (int(blockIdx.x) / nunit) % NWV;  // 64-channel group
    const int sg = int(blockIdx.x) / (nunit * NWV);  // segment of the slab
    if (W.flag[unit]) return;
    const int h = unit % A.H;
    const size_t b = size_t(unit / A.H);
    const int T = A.T;
    const int lane = threadIdx.x & 63;
    const int i = 64 * wv + lane;
    const float mu = A.mu;
    const bf16_t* kin = static_cast<const bf16_t*>(A.k);
    const bf16_t* ain = static_cast<const bf16_t*>(A.alpha);
    const bf16_t* win = static_cast<const bf16_t*>(A.omega);
    const bf16_t* rin = static_cast<const bf16_t*>(A.r);
    // the slab's buffers (token t at row t - tb) and the per-token sums
    const float* partial = W.partial + size_t(unit) * W.slab * ntile * 4 * DK;
    const float* pbuf = W.pbuf + size_t(unit) * W.slab * DK;
    float* tsc = W.tsc + size_t(unit) * T * 8;
    const auto tokidx = [&](int t) { return (b * size_t(T) + size_t(t)) * size_t(A.H) + size_t(h); };
    const int s0 = tb + sg * SEGU, s1 = min(te, s0 + SEGU);
    const auto load = [&](UncTok& x, int t) {
        t = max(t, s0);
        const size_t tok = tokidx(t);
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
            const int tc = min(tile, ntile - 1);
            const float* src = partial + (size_t(t - tb) * ntile + tc) * 4 * DK + i;
            x.k[tile] = __builtin_nontemporal_load(&src[DK]);
            if (!MAPS) {
                x.q[tile] = __builtin_nontemporal_load(&src[0]);
                x.ks[tile] = __builtin_nontemporal_load(&src[2 * DK]);
                x.a[tile] = __builtin_nontemporal_load(&src[3 * DK]);
            }
            x.u[tile] = tsc[size_t(t) * 8 + tc];
        }
        x.d = tsc[size_t(t) * 8 + 2];
        if (GATE) x.sk = tsc[size_t(t) * 8 + 6];
        x.pp = __builtin_nontemporal_load(&pbuf[size_t(t - tb) * DK + i]);
        x.al = ain[tok * DK + i];
        x.kk = kin[tok * DK + i];
        x.w = win[tok * DK + i];
        x.r = rin[tok];
    };
    const auto mapslot = [&](int s) { return W.maps + ((size_t(unit) * W.maxseg + s) * DK + i) * 2; };
    // dp carried between slabs: slab j reads what slab j + 1 left in buffer
    // (j + 1) & 1 and leaves its own in buffer j & 1
    const size_t cstride = size_t(nunit) * DK;
    float dp = 0.f, fa = 1.f, fb = 0.f;  // OUTPUTS: the carried dp; MAPS: dp_t = fa dp_in + fb
    if (!MAPS) {
        if (te == T) dp = A.dp_T ? A.dp_T[size_t(unit) * DK + i] : 0.f;
        else dp = W.dpc[size_t((slab + 1) & 1) * cstride + size_t(unit) * DK + i];
        for (int s = nseg - 1; s > sg; --s) {
            const float* m = mapslot(s);
            dp = fmaf(m[0], dp, m[1]);
        }
    }
    const float dpin = dp;
    const auto step = [&](int t, const UncTok& x) {
        const bool two = ntile > 1;
        const float gk = x.k[0] + (two ? x.k[1] : 0.f);
        const float u = x.u[0] + (two ? x.u[1] : 0.f);
        float al = bf1(x.al), kk = bf1(x.kk), w = bf1(x.w), rt = bf1(x.r);
        float ga_z = 1.f, gw_z = 1.f;  // (gated) the gates' derivatives at z
        if (GATE) {
            // the gated layer's values (as the gated forward forms them);
            // sigmoid' = sigmoid(z) sigmoid(-z) (no cancellation in
            // 1 - sigmoid), softplus' = sigmoid
            const float za = al, zw = w;
            al = gate_sigmoid(za);
            w = gate_softplus(zw);
            rt = kGateRMin + gate_softplus(rt);
            kk *= x.sk;
            if (!MAPS) {
                ga_z = al * gate_sigmoid(-za);
                gw_z = gate_sigmoid(zw);
            }
        }
        const size_t tok = tokidx(t);
        const float ph = al * al * x.pp + w;
        const float inv = 1.0f / x.d;
        const float dd = -u * inv * inv;
        const float mr = mu / rt;
        const float k2 = kk * kk;
        const float den = 1.0f + mr * k2 * ph;
        if (MAPS) {
            const float f = al * al / (den * den);
            fa *= f;
            fb = fmaf(f, fb, al * al * (gk * kk * inv + dd * k2));
            return;
        }
        const float gq = x.q[0] + (two ? x.q[1] : 0.f);
        const float gks = x.ks[0] + (two ? x.ks[1] : 0.f), ga = x.a[0] + (two ? x.a[1] : 0.f);
        const float pn = ph / den;
        const float du = -dp * pn * pn;
        const float dph = dp / (den * den) + gk * kk * inv + dd * k2;
        __builtin_nontemporal_store(gq, &A.dq[tok * DK + i]);
        __builtin_nontemporal_store(gks + gk * ph * inv + 2.0f * dd * ph * kk + 2.0f * du * mr * kk, &A.dk_[tok * DK + i]);
        // (gated: the gradients of the pre-activations)
        __builtin_nontemporal_store(GATE ? (ga + 2.0f * dph * al * x.pp) * ga_z : ga + 2.0f * dph * al * x.pp, &A.dalpha[tok * DK + i]);
        __builtin_nontemporal_store(GATE ? dph * gw_z : dph, &A.domega[tok * DK + i]);
        dp = dph * al * al;
        float dr = -du * mr * k2 / rt;
        dr = sum16(dr);
        dr = halve16(dr, dr);
        dr = halve32(dr, dr);
        if (lane == 0) {
            tsc[size_t(t) * 8 + 4 + wv] = dr;
            if (wv == 0) tsc[size_t(t) * 8 + 3] = dd;
        }
    };
    UncTok ring[PFU];
#pragma unroll
    for (int s = 0; s < PFU - 1; ++s) load(ring[s], max(s1 - 1 - s, s0));
    for (int t = s1 - 1; t >= s0; t -= PFU) {
#pragma unroll
        for (int s = 0; s < PFU; ++s) {
            load(ring[(s + PFU - 1) % PFU], max(t - s - (PFU - 1), s0));  // PFU - 1 tokens ahead
            if (t - s >= s0) step(t - s, ring[s]);
        }
    }
    if (MAPS) {
        float* m = mapslot(sg);
        m[0] = fa;
        m[1] = fb;
    } else if (sg == 0) {
        if (tb == 0) {
            A.dp0[size_t(unit) * DK + i] = dp;
        } else {
            const float* m = mapslot(0);
            W.dpc[size_t(slab & 1) * cstride + size_t(unit) * DK + i] = fmaf(m[0], dpin, m[1]);
        }
    }
}

// dr = dd + the waves' shares (one thread per token of a (batch, head) pair);
// GATE: times softplus' = sigmoid at the pre-activation
template <int DK, bool GATE>
__global__ void __launch_bounds__(256) kdn_backward_dr_kernel(BwdArgs A, ChunkWs W) {
    const int unit = int(blockIdx.y);
    const int t = int(blockIdx.x) * 256 + int(threadIdx.x);
    if (W.flag[unit] || t >= A.T) return;
    const float* ts = W.tsc + (size_t(unit) * A.T + t) * 8;
    float dr = ts[3];
#pragma unroll
    for (int w = 0; w < DK / 64; ++w) dr += ts[4 + w];
    const size_t b = size_t(unit / A.H);
    const size_t tok = (b * size_t(A.T) + size_t(t)) * size_t(A.H) + size_t(unit % A.H);
    if (GATE) dr *= gate_sigmoid(bf1(static_cast<const bf16_t*>(A.r)[tok]));
    A.dr[tok] = dr;
}

template <int DK, bool GATE>
hipError_t launch_unc_chunk_t(const BwdArgs& a, const ChunkWs& w, int slab, hipStream_t stream) {
    const int units = a.B * a.H;
    const int tb = slab * w.slab, te = std::min(a.T, tb + w.slab);
    const int nseg = (te - tb + SEGU - 1) / SEGU;
    const dim3 grid(unsigned(units * (DK / 64) * nseg));
    if (nseg > 1 || tb > 0)
        hipLaunchKernelGGL((kdn_backward_unc_chunk_kernel<DK, true, GATE>), grid, dim3(64), 0, stream, a, w, slab, tb,
                           te, nseg);
    hipLaunchKernelGGL((kdn_backward_unc_chunk_kernel<DK, false, GATE>), grid, dim3(64), 0, stream, a, w, slab, tb, te,
                       nseg);
    return hipGetLastError();
}

template <bool GATE>
hipError_t launch_chunk_t(const BwdArgs& a, const ChunkWs& w, int slab, hipStream_t stream) {
    const unsigned units = unsigned(long(a.B) * a.H);
    const unsigned grid = units * unsigned(a.dv / TILE);
    const int nchunks = (a.T + L - 1) / L;
    const int c_lo = slab * (w.slab / L), c_hi = std::min(nchunks, c_lo + w.slab / L);
    if (a.dk == 128)
        hipLaunchKernelGGL((kdn_backward_chunk_kernel<128, GATE>), dim3(grid), dim3(NTH), 0, stream, a, w, c_lo, c_hi);
    else if (a.dk == 64)
        hipLaunchKernelGGL((kdn_backward_chunk_kernel<64, GATE>), dim3(grid), dim3(NTH), 0, stream, a, w, c_lo, c_hi);
    else
        return hipErrorNotSupported;
    return hipGetLastError();
}

// region sizes of the chunked backward's workspace (ChunkWs order)
struct ChunkSizes {
    size_t b[9];
    size_t total() const {
        size_t t = 0;
        for (size_t x : b) t += (x + 255) & ~size_t(255);
        return t;
    }
};

ChunkSizes chunk_sizes(int B, int T, int H, int dk, int dv, int slab) {
    const size_t U = size_t(B) * size_t(H), nt = size_t(dv) / TILE, nch = (size_t(T) + L - 1) / L;
    const size_t S = size_t(slab), maxseg = size_t((slab + SEGU - 1) / SEGU), f = sizeof(float);
    return {{U * sizeof(int), U * nt * nch * dk * TILE * sizeof(uint16_t), U * nch * dk * f, U * size_t(T) * 8 * f,
             U * maxseg * dk * 2 * f, 2 * U * dk * f, U * size_t(dk) * dv * f, U * S * nt * 4 * dk * f,
             U * S * dk * f}};
}

// the shortest slab: about 64k token-heads of per-token buffers (512 tokens
// at B = 8, H = 16), at most the sequence
int chunk_min_slab(int B, int T, int H) {
    const long units = std::max(1L, long(B) * H);
    long s = (65536 + units - 1) / units;
    s = std::max(512L, (s + 511) / 512 * 512);
    const long tr = (long(T) + L - 1) / L * L;
    return int(std::min(s, tr));
}

}  // namespace

bool chunk_workspace(int B, int T, int H, int dk, int dv, void* work, size_t bytes, ChunkWs* out) {
    if (T <= 0) return false;
    const int tr = (T + L - 1) / L * L;
    int slab = chunk_min_slab(B, T, H);
    if (chunk_sizes(B, T, H, dk, dv, slab).total() > bytes) return false;
    // the longest slab that fits (fewer launches): the whole sequence, else a
    // multiple of SEGU
    for (int s2 = tr; s2 > slab; s2 = (s2 / 2 + SEGU - 1) / SEGU * SEGU)
        if (chunk_sizes(B, T, H, dk, dv, s2).total() <= bytes) {
            slab = s2;
            break;
        }
    const ChunkSizes z = chunk_sizes(B, T, H, dk, dv, slab);
    char* p = static_cast<char*>(work);
    char* reg[9];
    for (int j = 0; j < 9; ++j) {
        reg[j] = p;
        p += (z.b[j] + 255) & ~size_t(255);
    }
    out->flag = reinterpret_cast<int*>(reg[0]);
    out->cks = reinterpret_cast<uint16_t*>(reg[1]);
    out->ckp = reinterpret_cast<float*>(reg[2]);
    out->tsc = reinterpret_cast<float*>(reg[3]);
    out->maps = reinterpret_cast<float*>(reg[4]);
    out->dpc = reinterpret_cast<float*>(reg[5]);
    out->dsc = reinterpret_cast<float*>(reg[6]);
    out->partial = reinterpret_cast<float*>(reg[7]);
    out->pbuf = reinterpret_cast<float*>(reg[8]);
    out->slab = slab;
    out->nslab = (T + slab - 1) / slab;
    out->maxseg = (slab + SEGU - 1) / SEGU;
    out->rest = reg[1];
    out->rest_bytes = bytes - size_t(reg[1] - reg[0]);
    return true;
}

size_t chunk_workspace_min_bytes(int B, int T, int H, int dk, int dv) {
    return chunk_sizes(B, T, H, dk, dv, chunk_min_slab(B, T, H)).total();
}

hipError_t launch_backward_unc_chunk(const BwdArgs& a, const ChunkWs& w, int slab, hipStream_t stream) {
    if (a.dk == 128)
        return a.gates ? launch_unc_chunk_t<128, true>(a, w, slab, stream)
                       : launch_unc_chunk_t<128, false>(a, w, slab, stream);
    if (a.dk == 64)
        return a.gates ? launch_unc_chunk_t<64, true>(a, w, slab, stream)
                       : launch_unc_chunk_t<64, false>(a, w, slab, stream);
    return hipErrorNotSupported;
}

hipError_t launch_backward_chunk(const BwdArgs& a, const ChunkWs& w, int slab, hipStream_t stream) {
    return a.gates ? launch_chunk_t<true>(a, w, slab, stream) : launch_chunk_t<false>(a, w, slab, stream);
}

hipError_t launch_backward_dr(const BwdArgs& a, const ChunkWs& w, hipStream_t stream) {
    const dim3 grid(unsigned((a.T + 255) / 256), unsigned(a.B * a.H));
    if (a.dk == 128) {
        if (a.gates) hipLaunchKernelGGL((kdn_backward_dr_kernel<128, true>), grid, dim3(256), 0, stream, a, w);
        else hipLaunchKernelGGL((kdn_backward_dr_kernel<128, false>), grid, dim3(256), 0, stream, a, w);
    } else if (a.dk == 64) {
        if (a.gates) hipLaunchKernelGGL((kdn_backward_dr_kernel<64, true>), grid, dim3(256), 0, stream, a, w);
        else hipLaunchKernelGGL((kdn_backward_dr_kernel<64, false>), grid, dim3(256), 0, stream, a, w);
    } else {
        return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace kdn
