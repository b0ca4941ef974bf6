// kdn_recurrent_core.h -- one wave's share of the token-by-token KDN
// recurrence on gfx950: 32 value columns of one (batch, head) pair, the
// memory S of those columns in registers.  Used by the recurrent kernel
// (whole sequences, the decode step) and by the chunked kernel, which
// finishes a sequence with it from the first chunk whose decays leave the
// chunked form's range.
//
// Lane = (row group rg in 0..7, column quad cq in 0..7): the lane holds rows
// rg, rg + 8, ... (d_k / 8 rows) of 4 consecutive columns, so every column
// reduction over the key dimension is a reduction inside the wave.
//
// Per token ("Kalman Delta Networks: Uncertainty-aware Associative Memory",
// summary page, method steps 2-5; isotropic variant per the closing sentence
// of that section, with a scalar decay or, in its general form, one decay per
// key channel and the trace projection a = mean_i alpha_i^2 for the
// uncertainty scalar):
//   the wave runs the per-channel part (lane owns channels lane and
//   lane + 64): predict p_hat, gain denominator r + sum p_hat k^2, kappa,
//   kappa^T q, posterior p; it stages (alpha_i, k_i, q_i, kappa_i) in its own
//   slice of LDS;
//   then on its columns: S_hat = diag(alpha) S, the two key-dimension dot
//   products S_hat^T k and S_hat^T q in one pass, innovation
//   delta = v - S_hat^T k, readout o = S_hat^T q + (kappa^T q) delta (the
//   post-write readout expanded), and the write S = S_hat + kappa delta^T.
#pragma once

#include "kdn_device.h"
#include "kdn_gates.h"

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace kdn {
namespace rec {

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

// sum over the wave, in every lane: DPP inside 16-lane rows, then the row
// swaps (no LDS round trip on the per-token dependency chain)
__device__ __forceinline__ float wave_sum(float x) {
    x = dev::sum16(x);
    x = dev::halve16(x, x);
    return dev::halve32(x, x);
}

// LDS written by some lanes of a wave and read by other lanes of the same
// wave: order the accesses at wavefront scope (no workgroup barrier).  One
// wave's LDS operations execute in order, so waiting for this wave's own LDS
// traffic and keeping the compiler from moving memory accesses across is
// enough; a memory fence would also wait for every global load in flight.
__device__ __forceinline__ void wave_lds_sync_rec() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Where one wave's tokens live.  Token t of the sequence is row tok0 + t of
// the [tokens, H] grid; the wave's columns are col0 .. col0 + 31 of d_v.
template <typename Tin>
struct RecIO {
    const Tin* q;
    const Tin* k;
    const Tin* v;  // not read when run_tokens is instantiated with VZ (v = 0)
    const Tin* alpha;
    const Tin* omega;
    const Tin* r;
    Tin* o;
    float mu;
    int H, dv;
    int h;
    size_t tok0;
    int col;   // first of this lane's four columns (col0 + 4 cq)
    int ng;    // entries of r per head-token (noise groups; 1 unless GR)
    int grp;   // this wave's noise group (GR)
    bool gates;
};

// Tokens [t_begin, t_end) of the sequence.  S: rows rg + 8 m, columns
// col .. col + 3; p: channels lane + 64 c (diagonal) or pb (isotropic forms).
// chan: this wave's own LDS slice of d_k float4.  VZ: v = 0 (columns that
// carry a state transition; a.v is not read).
template <int DK, int VAR, typename Tin, bool GR, bool VZ = false>
__device__ __forceinline__ void run_tokens(const RecIO<Tin>& a, float (&S)[DK / 8][4], float (&p)[DK / 64],
                                           float& pb, float4* chan, int t_begin, int t_end) {
    constexpr bool ISO = VAR != 0;   // one uncertainty scalar per head
    constexpr bool CHAN = VAR != 1;  // one decay per key channel
    constexpr int CPL = DK / 64;     // channels per lane
    constexpr int RPT = DK / 8;      // memory rows per lane
    const int lane = threadIdx.x & 63;
    const int rg = lane >> 3;
    const float inv_dk = 1.0f / float(DK);
    for (int t = t_begin; t < t_end; ++t) {
        const size_t tok = (a.tok0 + size_t(t)) * size_t(a.H) + size_t(a.h);
        float rt = to_f32(a.r[GR ? tok * a.ng + a.grp : tok]);
        // gates: alpha, omega and r arrive as pre-activations
        if (a.gates) rt = kGateRMin + gate_softplus(rt);
        float kk[CPL], qq[CPL], aa[CPL], kap[CPL];
        float mq;  // kappa^T q
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            kk[c] = to_f32(a.k[tok * DK + lane + 64 * c]);
            qq[c] = to_f32(a.q[tok * DK + lane + 64 * c]);
        }
        if (a.gates) {
            // the prologue's normalisation of q and k (over the d_k channels)
            float nk = 0.f, nq = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                nk = fmaf(kk[c], kk[c], nk);
                nq = fmaf(qq[c], qq[c], nq);
            }
            const float sk = inv_norm(wave_sum(nk)), sq = inv_norm(wave_sum(nq));
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                kk[c] *= sk;
                qq[c] *= sq;
            }
        }
        if (ISO) {
            // trace-projected predict b_hat = a b + omega / d_k; a = alpha^2,
            // or with per-channel decay the mean of alpha_i^2 over the channels
            float w = to_f32(a.omega[tok]);
            if (a.gates) w = gate_softplus(w);
            float a2 = 0.f, n = 0.f, kq = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                aa[c] = CHAN ? to_f32(a.alpha[tok * DK + lane + 64 * c]) : to_f32(a.alpha[tok]);
                if (a.gates) aa[c] = gate_sigmoid(aa[c]);
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
            pb = bh / (1.0f + (a.mu / (float(DK) * rt)) * n * bh);
        } else {
            float ph[CPL];
            float s = 0.f, kq = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                aa[c] = to_f32(a.alpha[tok * DK + lane + 64 * c]);
                float w = to_f32(a.omega[tok * DK + lane + 64 * c]);
                if (a.gates) {
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
            const float mr = a.mu / rt;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                kap[c] = ph[c] * kk[c] * inv;
                p[c] = ph[c] / (1.0f + mr * kk[c] * kk[c] * ph[c]);
            }
            mq = kq * inv;
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) chan[lane + 64 * c] = make_float4(aa[c], kk[c], qq[c], kap[c]);
        wave_lds_sync_rec();

        float A[4] = {0.f, 0.f, 0.f, 0.f}, Bq[4] = {0.f, 0.f, 0.f, 0.f};
        float kr[RPT];
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const float4 c4 = chan[rg + 8 * m];
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
        for (int j = 0; j < 4; ++j) d[j] = (VZ ? 0.f : to_f32(a.v[tok * a.dv + a.col + j])) - A[j];
#pragma unroll
        for (int m = 0; m < RPT; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[m][j] += kr[m] * d[j];
        if (rg == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) from_f32(a.o + tok * a.dv + a.col + j, Bq[j] + mq * d[j]);
        }
        wave_lds_sync_rec();  // chan is rewritten by the next token
    }
}

}  // namespace rec
}  // namespace kdn
