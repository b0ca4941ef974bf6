// kdn_split.hip -- the diagonal forward of a long sequence cut into segments
// that run concurrently (for batches too small to fill the device with one
// workgroup per (batch, head) and column tile).
//
// Method ("Kalman Delta Networks: Uncertainty-aware Associative Memory",
// summary page, method steps 2-5).  Both recurrences of a (batch, head) pair
// compose across a cut of the sequence:
//  - the uncertainty: each token's update of p_i is a Mobius map, the 2 x 2
//    matrix [[a, w], [u a, 1 + u w]] with a = alpha_i^2, w = omega_i,
//    u = (mu / r) k_i^2 (step 5), so a segment's effect on p_i is the
//    product of its tokens' matrices, and the uncertainty entering segment g
//    is p0 carried through the products of segments 0 .. g-1;
//  - the memory: given the gains, S_t = A_t S_{t-1} + B_t is affine in S
//    (A_t = (I - kappa_t k_t^T) diag(alpha_t), B_t = kappa_t v_t^T, step 4),
//    so over segment g, S_end = Phi_g S_start + Psi_g and every output is
//    o_t = o_t^Psi + (Phi_t^T q_t)^T S_start, with Phi_t the transition from
//    the segment's start to token t.
// The chunked kernel runs every segment at once from S = 0 on the v columns
// (giving Psi_g and o^Psi) and from S = I on d_k extra columns with v = 0
// (giving Phi_g and o^Phi_t = Phi_t^T q_t); the first segment starts from S0
// and needs no identity columns.  Then
//   S_{g+1} = Phi_g S_g + Psi_g  (kdn_split_compose_kernel, fp32, sequential
//   over the segments) and o_t += (o^Phi_t)^T S_g for the tokens of segments
//   g >= 1 (kdn_split_correct_kernel, matrix cores, S_g rounded to bf16).
#include "kdn_device.h"
#include "kdn_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>

namespace kdn {
namespace {

using namespace dev;

constexpr int SUB = 256;  // tokens per sub-segment of the Mobius products
constexpr int TB = 256;   // tokens per workgroup of the output correction

__device__ __forceinline__ float4 mob_mul(float4 m, float4 x) {
    // m x for 2 x 2 matrices stored (00, 01, 10, 11), scaled so that the 11
    // entry is about 1: a Mobius map does not change under scaling, so the
    // scale only keeps the entries in range and need not be exact
    const float y00 = fmaf(m.x, x.x, m.y * x.z), y01 = fmaf(m.x, x.y, m.y * x.w);
    const float y10 = fmaf(m.z, x.x, m.w * x.z), y11 = fmaf(m.z, x.y, m.w * x.w);
    const float s = __builtin_amdgcn_rcpf(y11);
    return make_float4(y00 * s, y01 * s, y10 * s, y11 * s);
}

// Products of the token maps of sub-segment `sub` of segment g for
// (batch, head) unit: thread x takes channels 4 c .. 4 c + 3 (c = x % (DK / 4))
// of one sub-segment (8-byte loads of each input row; four independent
// products); later tokens multiply from the left.
template <int DK>
__global__ void __launch_bounds__(64) kdn_split_mob_sub_kernel(const bf16_t* __restrict__ k,
                                                               const bf16_t* __restrict__ alpha,
                                                               const bf16_t* __restrict__ omega,
                                                               const bf16_t* __restrict__ r, float mu, int T, int H,
                                                               int seg, int nseg, int nsub, int total,
                                                               float4* __restrict__ out) {
    constexpr int NQ = DK / 4;  // channel quads
    const int x = blockIdx.x * 64 + threadIdx.x;
    if (x >= total) return;
    const int cq = x % NQ;
    const int sub = (x / NQ) % nsub;
    const int g = (x / (NQ * nsub)) % nseg;
    const int unit = x / (NQ * nsub * nseg);
    const int b = unit / H, h = unit % H;
    const int t0 = g * seg + sub * SUB;
    const int t1 = min(min(t0 + SUB, (g + 1) * seg), T);
    float4 P[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) P[c] = make_float4(1.f, 0.f, 0.f, 1.f);
    // Batches of U tokens in two register sets: the next batch's loads are
    // issued before this batch's maps are applied, so the composition runs
    // while they are in flight.  Loads past the sub-segment read its last
    // token (clamped) and are not applied.
    constexpr int U = 8;
    struct Batch {
        u2 al[U], w[U], kk[U];
        float rr[U];
    };
    const auto load = [&](Batch& B, int tb) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const size_t tok = (size_t(b) * T + min(tb + j, t1 - 1)) * H + h;
            B.al[j] = *reinterpret_cast<const u2*>(alpha + tok * DK + 4 * cq);
            B.w[j] = *reinterpret_cast<const u2*>(omega + tok * DK + 4 * cq);
            B.kk[j] = *reinterpret_cast<const u2*>(k + tok * DK + 4 * cq);
            B.rr[j] = bf1(r[tok]);
        }
    };
    const auto apply = [&](const Batch& B, int tb) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
            if (tb + j < t1) {
                const float mr = mu / B.rr[j];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t wa = B.al[j][c >> 1], ww = B.w[j][c >> 1], wk = B.kk[j][c >> 1];
                    const float a = (c & 1) ? bf_hi(wa) : bf_lo(wa), om = (c & 1) ? bf_hi(ww) : bf_lo(ww);
                    const float kv = (c & 1) ? bf_hi(wk) : bf_lo(wk);
                    const float u = mr * kv * kv, a2 = a * a;
                    P[c] = mob_mul(make_float4(a2, om, u * a2, fmaf(u, om, 1.f)), P[c]);
                }
            }
        }
    };
    Batch A, B;
    load(A, t0);
    for (int tb = t0; tb < t1; tb += 2 * U) {
        load(B, tb + U);
        apply(A, tb);
        load(A, tb + 2 * U);
        apply(B, tb + U);
    }
    float4* dst = out + ((size_t(unit) * nseg + g) * nsub + sub) * DK + 4 * cq;
#pragma unroll
    for (int c = 0; c < 4; ++c) dst[c] = P[c];
}

// The segments' products from their sub-segments' (in token order), loaded
// 16 at a time ahead of their use.
template <int DK>
__global__ void __launch_bounds__(DK) kdn_split_mob_combine_kernel(const float4* __restrict__ sub, int nseg,
                                                                   int nsub, float4* __restrict__ mob) {
    const int i = threadIdx.x;
    const size_t ug = blockIdx.x;  // unit * nseg + g
    float4 P = make_float4(1.f, 0.f, 0.f, 1.f);
    constexpr int U = 16;
    for (int s0 = 0; s0 < nsub; s0 += U) {
        float4 m[U];
#pragma unroll
        for (int j = 0; j < U; ++j) m[j] = sub[(ug * nsub + min(s0 + j, nsub - 1)) * DK + i];
#pragma unroll
        for (int j = 0; j < U; ++j)
            if (s0 + j < nsub) P = mob_mul(m[j], P);
    }
    mob[ug * DK + i] = P;
}

// S at every segment's start: S_1 = the first segment's end state, then
// S_{g+1} = Phi_g S_g + Psi_g.  One workgroup per (batch, head) and 16 value
// columns; thread (row tid / 2, columns 8 (tid & 1) .. + 7).  S_g (g >= 1)
// go to sinT as bf16, transposed ([value column][d_k], the correction's
// operand), the last to S_T.
template <int DK>
__global__ void __launch_bounds__(2 * DK) kdn_split_compose_kernel(const float* __restrict__ sseg, int nseg, int DV,
                                                                   bf16_t* __restrict__ sinT, float* __restrict__ S_T) {
    __shared__ float S[DK][16];
    const int row = threadIdx.x >> 1, c0 = 8 * (threadIdx.x & 1);
    const int nblk = DV / 16;
    const int unit = blockIdx.x / nblk, col0 = 16 * (blockIdx.x % nblk);
    const int SW = DV + DK;  // row stride of the segment states
    const float* s0 = sseg + size_t(unit) * nseg * DK * SW;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = s0[size_t(row) * SW + col0 + c0 + j];
    for (int g = 1; g < nseg; ++g) {
        __syncthreads();  // the previous step's reads of S are done
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            S[row][c0 + j] = acc[j];
            sinT[((size_t(unit) * nseg + g) * DV + col0 + c0 + j) * DK + row] = to_bf(acc[j]);
        }
        __syncthreads();
        const float* sg = sseg + (size_t(unit) * nseg + g) * DK * SW;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = sg[size_t(row) * SW + col0 + c0 + j];  // Psi_g
        const float* phi = sg + size_t(row) * SW + DV;                                // row of Phi_g
        for (int kk = 0; kk < DK; kk += 4) {
            const float4 f = *reinterpret_cast<const float4*>(phi + kk);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                acc[j] = fmaf(f.x, S[kk][c0 + j], acc[j]);
                acc[j] = fmaf(f.y, S[kk + 1][c0 + j], acc[j]);
                acc[j] = fmaf(f.z, S[kk + 2][c0 + j], acc[j]);
                acc[j] = fmaf(f.w, S[kk + 3][c0 + j], acc[j]);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) S_T[(size_t(unit) * DK + row) * DV + col0 + c0 + j] = acc[j];
}

// o_t += (o^Phi_t)^T S_g for the tokens of segment g >= 1: per workgroup one
// (batch, head), one segment and TB of its tokens; wave w takes the 16-token
// row tiles w, w + 4, ... and every value column.  On matrix cores with bf16
// operands: A = S_g^T (value column x d_k, from LDS), B = the tokens' o^Phi
// rows, so each lane's accumulator is 4 consecutive value columns of one token.
template <int DK, int DV>
__global__ void __launch_bounds__(256) kdn_split_correct_kernel(const bf16_t* __restrict__ ophi,
                                                                const bf16_t* __restrict__ sinT,
                                                                bf16_t* __restrict__ o, int T, int H, int seg, int nseg) {
    constexpr int P = DK + 8;  // pitch of the S^T rows (bf16): 16-byte aligned, rows on different banks
    __shared__ __align__(16) bf16_t St[DV * P];
    const int nblk = (seg + TB - 1) / TB;
    const int blk = blockIdx.x % nblk;
    const int g = 1 + (blockIdx.x / nblk) % (nseg - 1);
    const int unit = blockIdx.x / (nblk * (nseg - 1));
    const int b = unit / H, h = unit % H;
    const int tseg = g * seg, tend = min(T, tseg + seg);
    const int tb = tseg + TB * blk;
    if (tb >= tend) return;
    const bf16_t* sg = sinT + (size_t(unit) * nseg + g) * DV * DK;
    for (int x = threadIdx.x; x < DV * DK / 8; x += 256) {
        const int col = x / (DK / 8), k8 = 8 * (x % (DK / 8));
        *reinterpret_cast<u4*>(&St[col * P + k8]) = *reinterpret_cast<const u4*>(sg + size_t(col) * DK + k8);
    }
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = (lane >> 4) * 4, kg8 = (lane >> 4) * 8;
    constexpr int KS = DK / 32;
    constexpr int NTW = TB / 64;  // 16-token row tiles per wave: w, w + 4, ...
    // One row tile's operands: the tokens' o^Phi rows and their current
    // outputs, loaded a tile ahead of its products (tokens past the segment
    // read its last token and are not written).
    struct Tile {
        b8 bo[KS];
        u2 cur[DV / 16];
    };
    const auto load = [&](Tile& X, int rt) {
        const int tn = min(tb + 16 * rt + n, tend - 1);
        const size_t tok = (size_t(b) * T + tn) * H + h;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) X.bo[kk] = *reinterpret_cast<const b8*>(ophi + tok * DK + 32 * kk + kg8);
#pragma unroll
        for (int ct = 0; ct < DV / 16; ++ct) X.cur[ct] = *reinterpret_cast<const u2*>(o + tok * DV + 16 * ct + g4);
    };
    const auto apply = [&](const Tile& X, int rt) {
        // every lane takes part in the products (the matrix cores read the
        // operands of the whole wave); only tokens inside the segment store
        const int tn = tb + 16 * rt + n;  // this lane's token (B operand column, output row)
        const bool ok = tn < tend;
        bf16_t* orow = o + ((size_t(b) * T + min(tn, tend - 1)) * H + h) * DV;
#pragma unroll
        for (int ct = 0; ct < DV / 16; ++ct) {
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const b8 as = *reinterpret_cast<const b8*>(&St[(16 * ct + n) * P + 32 * kk + kg8]);
                acc = mfma32(as, X.bo[kk], acc);
            }
            // acc[e]: value column 16 ct + g4 + e of token tn
            const float o0 = bf_lo(X.cur[ct][0]) + acc[0], o1 = bf_hi(X.cur[ct][0]) + acc[1];
            const float o2 = bf_lo(X.cur[ct][1]) + acc[2], o3 = bf_hi(X.cur[ct][1]) + acc[3];
            if (ok) *reinterpret_cast<u2*>(orow + 16 * ct + g4) = u2{pack2(o0, o1), pack2(o2, o3)};
        }
    };
    Tile X0, X1;
    load(X0, wave);
#pragma unroll
    for (int i = 0; i < NTW; i += 2) {
        if (i + 1 < NTW) load(X1, wave + 4 * (i + 1));
        apply(X0, wave + 4 * i);
        if (i + 2 < NTW) load(X0, wave + 4 * (i + 2));
        if (i + 1 < NTW) apply(X1, wave + 4 * (i + 1));
    }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct SplitLayout {
    int nseg = 1, seg = 0, nsub = 1;
    size_t off_sub = 0, off_mob = 0, off_ophi = 0, off_sseg = 0, off_sin = 0, bytes = 0;
};

SplitLayout split_layout(int B, int T, int H, int dk, int dv, int nseg) {
    SplitLayout L;
    if (nseg < 2 || T < 64) return L;
    const int per = (T + nseg - 1) / nseg;
    L.seg = (per + 31) / 32 * 32;
    L.nseg = (T + L.seg - 1) / L.seg;
    if (L.nseg < 2) {
        L.nseg = 1;
        return L;
    }
    L.nsub = (L.seg + SUB - 1) / SUB;
    const size_t units = size_t(B) * H;
    size_t off = 0;
    L.off_sub = off;
    off = align256(off + units * L.nseg * L.nsub * dk * 16);
    L.off_mob = off;
    off = align256(off + units * L.nseg * dk * 16);
    L.off_ophi = off;
    off = align256(off + size_t(B) * T * H * dk * 2);
    L.off_sseg = off;
    off = align256(off + units * L.nseg * dk * (dv + dk) * 4);
    L.off_sin = off;
    off = align256(off + units * L.nseg * dk * dv * 2);
    L.bytes = off;
    return L;
}

template <int DK>
hipError_t launch_split_dk(const FwdArgs& a, const SplitLayout& L, unsigned char* ws, hipStream_t stream) {
    const int units = a.B * a.H;
    float4* sub = reinterpret_cast<float4*>(ws + L.off_sub);
    float4* mob = reinterpret_cast<float4*>(ws + L.off_mob);
    bf16_t* ophi = reinterpret_cast<bf16_t*>(ws + L.off_ophi);
    float* sseg = reinterpret_cast<float*>(ws + L.off_sseg);
    bf16_t* sinT = reinterpret_cast<bf16_t*>(ws + L.off_sin);
    const int nthr = units * L.nseg * L.nsub * (DK / 4);
    hipLaunchKernelGGL((kdn_split_mob_sub_kernel<DK>), dim3((nthr + 63) / 64), dim3(64), 0, stream,
                       static_cast<const bf16_t*>(a.k), static_cast<const bf16_t*>(a.alpha),
                       static_cast<const bf16_t*>(a.omega), static_cast<const bf16_t*>(a.r), a.mu, a.T, a.H, L.seg,
                       L.nseg, L.nsub, nthr, sub);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((kdn_split_mob_combine_kernel<DK>), dim3(units * L.nseg), dim3(DK), 0, stream, sub, L.nseg,
                       L.nsub, mob);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = launch_chunked_segments(a, L.seg, L.nseg, reinterpret_cast<const float*>(mob), ophi, sseg, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((kdn_split_compose_kernel<DK>), dim3(units * (a.dv / 16)), dim3(2 * DK), 0, stream, sseg,
                       L.nseg, a.dv, sinT, a.S_T);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const unsigned grid = unsigned(units) * unsigned(L.nseg - 1) * unsigned((L.seg + TB - 1) / TB);
    bf16_t* o = static_cast<bf16_t*>(a.o);
    if (a.dv == 128)
        hipLaunchKernelGGL((kdn_split_correct_kernel<DK, 128>), dim3(grid), dim3(256), 0, stream, ophi, sinT, o,
                           a.T, a.H, L.seg, L.nseg);
    else
        hipLaunchKernelGGL((kdn_split_correct_kernel<DK, 64>), dim3(grid), dim3(256), 0, stream, ophi, sinT, o,
                           a.T, a.H, L.seg, L.nseg);
    return hipGetLastError();
}

}  // namespace

int split_segments(int B, int T, int H, int dk, int dv, int requested, long cus) {
    if (requested > 0) return split_layout(B, T, H, dk, dv, requested).nseg;
    // as many segments as fill the device with one workgroup per CU, each
    // segment at least 2048 tokens
    const long per = long(B) * H * (dv / 64 + dk / 64);
    long n = per > 0 ? cus / per : 1;
    n = std::min<long>(n, std::max(1, T / 2048));
    n = std::min<long>(n, 16);
    return n >= 2 ? split_layout(B, T, H, dk, dv, int(n)).nseg : 1;
}

size_t split_workspace_bytes(int B, int T, int H, int dk, int dv, int nseg) {
    return split_layout(B, T, H, dk, dv, nseg).bytes;
}

hipError_t launch_split(const FwdArgs& a, int nseg, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const SplitLayout L = split_layout(a.B, a.T, a.H, a.dk, a.dv, nseg);
    if (L.nseg < 2) return launch_chunked(a, stream);
    if (!workspace || workspace_bytes < L.bytes) return hipErrorInvalidValue;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    return a.dk == 128 ? launch_split_dk<128>(a, L, ws, stream) : launch_split_dk<64>(a, L, ws, stream);
}

}  // namespace kdn
