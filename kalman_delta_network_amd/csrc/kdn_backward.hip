// kdn_backward.hip -- reverse-mode gradients of the KDN recurrence for gfx950.
//
// The forward token step (KDN summary page, method steps 2-5; isotropic forms
// per the closing sentence of that section) is
//   p_hat = alpha^2 p + omega,  kappa = p_hat k / (r + sum p_hat k^2),
//   S_hat = diag(alpha) S,  delta = v - S_hat^T k,  S' = S_hat + kappa delta^T,
//   o = S'^T q,  p' = p_hat / (1 + (mu / r) k^2 p_hat),
// and this kernel runs its adjoint backwards in time.  The adjoint splits in
// two coupled parts:
//   * the memory part, on the d_k x d_v cotangent dS, needs only kappa, alpha,
//     k, q from the uncertainty path:
//       dS += q dO^T;  d_delta = dS^T kappa (= dv);  d_kappa = dS delta;
//       dq = S' dO;  dS_hat = dS - k d_delta^T;  dk_mem = -S_hat d_delta;
//       dalpha_mem = rowsum(S (.) dS_hat);  dS <- diag(alpha) dS_hat;
//   * the uncertainty part, per key channel, needs d_kappa from the memory
//     part and carries dp backwards through the posterior, the gain and the
//     prediction (dk, dalpha, domega, dr).
//
// Two kernels.  The memory kernel takes one workgroup per (batch, head, 64
// value columns) with 8 waves: lane = (row group rg, column cq), holding rows
// rg + 8m of one column, so that each column reduction over the key
// dimension stays inside one wave (DPP within rows, row swaps across).  The
// uncertainty kernel takes one wave per (batch, head) (lane owns channels
// lane, lane + 64).  Every global load of the token loops is issued three
// tokens ahead into a ring of four buffers.
//
// The memory S_{t-1} is needed at every token of the reverse sweep.  A first
// forward sweep stores a checkpoint of (S, p) every SEG tokens in the
// workspace; then, segment by segment from the last, the memory waves re-run
// the segment's forward from its checkpoint, storing each token's S_{t-1} in
// a per-workgroup stash (workspace) and the token's (alpha, k, q, kappa) in
// LDS (and p_{t-1} in the workspace), and walk the segment backwards.  They
// reduce their four per-row partial sums (dq, d_kappa, dk_mem, dalpha_mem)
// over the lanes of a row with a reduce-scatter, then over the waves through
// LDS one token behind, and store the tile's sums per token in the
// workspace; the uncertainty kernel adds the tiles and runs its part
// backwards over the tokens.
//
// Each pair needs token_pair_bytes() of workspace.  The kernels take the
// pairs in rounds of as many as the workspace holds (all of them with
// backward_workspace_bytes()); pair slot0 + s of a round uses slot s.
#include "kdn_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>

namespace kdn {
namespace {

typedef uint16_t bf16_t;  // raw bfloat16 bits

constexpr int SEG = 32;  // tokens per checkpoint segment
constexpr int NC = 1;    // memory columns per lane
constexpr int SG = 4 / NC;  // memory rows per float4 of a snapshot
constexpr int PF = 4;       // prefetch ring: token loads are issued PF - 1 tokens ahead
constexpr int WCOLS = 8 * NC;  // memory columns per wave

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// Cross-lane exchanges without the LDS pipe: DPP within rows of 16 lanes
// and the gfx950 row-swap instructions across rows.  Each pair sums a + b
// on both sides, so every lane of a group ends with the same bits.
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7 - i within 8
constexpr int DPP_MIRROR = 0x140;      // lane i <-> 15 - i within 16
constexpr int DPP_ROR8 = 0x128;        // lane i <-> i ^ 8 within 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// x[l] + x[l ^ 16] and x[l] + x[l ^ 32] in every lane
__device__ __forceinline__ float add_xor16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// sum over the 64 lanes, in every lane
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp<DPP_XOR1>(x);
    x += dpp<DPP_XOR2>(x);
    x += dpp<DPP_HALF_MIRROR>(x);
    x += dpp<DPP_MIRROR>(x);
    return add_xor32(add_xor16(x));
}

// sum over the 8 row groups (lane bits 3..5) of a memory wave, in every lane
__device__ __forceinline__ float rowgroup_sum(float x) {
    x += dpp<DPP_ROR8>(x);
    return add_xor32(add_xor16(x));
}

__device__ __forceinline__ void wave_lds_sync() {
    // One wave's LDS operations execute in order, so waiting for this wave's
    // own LDS traffic and keeping the compiler from moving memory accesses
    // across is enough; a memory fence would also wait for every global load
    // still in flight (the next token's prefetch).
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Workgroup barrier for LDS data only: global loads in flight (prefetches)
// stay in flight across it.
__device__ __forceinline__ void block_lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// workspace floats per (batch, head, column tile of dv columns): S and p
// checkpoints (p once per memory wave, so that every lane reads back only
// what it wrote) and the stash
__host__ __device__ inline size_t unit_floats(int T, int dk, int dv) {
    const size_t nseg = (size_t(T) + SEG - 1) / SEG;
    const size_t nw = size_t(dv) / WCOLS;
    return nseg * (size_t(dk) * dv + nw * dk) + size_t(SEG) * dk * dv;
}

template <int DK, int DV>
struct BwdSmem {
    float4 seg_chan[SEG][DK];           // (alpha, k, q, kappa) of each token of the segment
    float part[2][4][DV / WCOLS][DK];   // per-wave row sums: dq, d_kappa, dk_mem, dalpha_mem
    float4 chan[DV / WCOLS][DK];        // forward staging, one slice per memory wave
};

// float4 index, within one memory snapshot, of rows m .. m + SG - 1 of
// thread tid: each wave owns RPT / SG blocks of 64 float4 (1 KB), one per row
// group, with the lanes contiguous, so every snapshot access is one coalesced
// 1 KB run per wave and the row groups of a thread differ by immediate offsets
template <int RPT>
__device__ __forceinline__ int snap_idx(int tid, int m) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    return (wave * (RPT / SG) + m / SG) * 64 + (tid & 63);
}

// rows m .. m + SG - 1 (all NC columns) of a lane's memory block as one float4
template <int RPT>
__device__ __forceinline__ float4 snap_pack(const float (&S)[RPT][NC], int m) {
    return make_float4(S[m + 0 / NC][0 % NC], S[m + 1 / NC][1 % NC], S[m + 2 / NC][2 % NC], S[m + 3 / NC][3 % NC]);
}
template <int RPT>
__device__ __forceinline__ void snap_unpack(float (&S)[RPT][NC], int m, float4 v) {
    S[m + 0 / NC][0 % NC] = v.x;
    S[m + 1 / NC][1 % NC] = v.y;
    S[m + 2 / NC][2 % NC] = v.z;
    S[m + 3 / NC][3 % NC] = v.w;
}

// One token's inputs as loaded (raw bf16 or fp32): a prefetch is converted
// where it is used, so that nothing waits for it earlier.
template <int DK, int VAR, typename Tin>
struct TokIn {
    static constexpr int CPL = DK / 64;
    Tin k[CPL], q[CPL], a[CPL], w[CPL];
    Tin r;
    Tin v[NC];
};

// GR: grouped observation noise, r [.., ngroups]; this tile's group is rg_off
template <int DK, int VAR, typename Tin, bool GR = false>
__device__ __forceinline__ void load_tok(TokIn<DK, VAR, Tin>& x, const BwdArgs& A, size_t tok, int lane,
                                         int col, int DVv, int ngroups = 1, int rg_off = 0) {
    constexpr int CPL = DK / 64;
    const Tin* q = static_cast<const Tin*>(A.q);
    const Tin* k = static_cast<const Tin*>(A.k);
    const Tin* v = static_cast<const Tin*>(A.v);
    const Tin* al = static_cast<const Tin*>(A.alpha);
    const Tin* om = static_cast<const Tin*>(A.omega);
    const Tin* r = static_cast<const Tin*>(A.r);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const size_t e = tok * DK + lane + 64 * c;
        x.k[c] = k[e];
        x.q[c] = q[e];
        x.a[c] = VAR == 1 ? al[tok] : al[e];
        x.w[c] = VAR == 0 ? om[e] : om[tok];
    }
    x.r = r[GR ? tok * size_t(ngroups) + size_t(rg_off) : tok];
#pragma unroll
    for (int j = 0; j < NC; ++j) x.v[j] = v[tok * DVv + col + j];
}

// One forward token on a memory wave's columns (the recurrent forward's
// arithmetic, without the readout).  Optionally records the token's
// (alpha, k, q, kappa) and p_{t-1} for the reverse sweep (wave 0) and the
// pre-token memory S_{t-1} in the stash (every memory wave).
template <int DK, int DV, int VAR, typename Tin>
__device__ __forceinline__ void fwd_token(const TokIn<DK, VAR, Tin>& x, float (&S)[DK / 8][NC],
                                          float (&p)[DK / 64], float& pb, float mu, float4* chanw,
                                          float4* rec_chan, float* rec_p, float4* stash_tok, int lane,
                                          int rg, int tid) {
    constexpr int CPL = DK / 64, RPT = DK / 8;
    constexpr bool ISO = VAR != 0;
    float xk[CPL], xq[CPL], xa[CPL], xw[CPL], xv[NC];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        xk[c] = to_f32(x.k[c]);
        xq[c] = to_f32(x.q[c]);
        xa[c] = to_f32(x.a[c]);
        xw[c] = to_f32(x.w[c]);
    }
    const float xr = to_f32(x.r);
#pragma unroll
    for (int j = 0; j < NC; ++j) xv[j] = to_f32(x.v[j]);
    float kap[CPL];
    if (ISO) {
        float a2 = 0.f, n = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            a2 += xa[c] * xa[c];
            n += xk[c] * xk[c];
        }
        a2 = VAR == 2 ? wave_sum(a2) * (1.0f / float(DK)) : xa[0] * xa[0];
        n = wave_sum(n);
        const float bh = a2 * pb + xw[0] * (1.0f / float(DK));
        const float beta = bh / (xr + bh * n);
#pragma unroll
        for (int c = 0; c < CPL; ++c) kap[c] = beta * xk[c];
        if (rec_p && lane == 0) rec_p[0] = pb;
        pb = bh / (1.0f + (mu / (float(DK) * xr)) * n * bh);
    } else {
        float ph[CPL];
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            ph[c] = xa[c] * xa[c] * p[c] + xw[c];
            s += ph[c] * xk[c] * xk[c];
        }
        s = wave_sum(s);
        const float inv = 1.0f / (xr + s);
        const float mr = mu / xr;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            kap[c] = ph[c] * xk[c] * inv;
            if (rec_p) rec_p[lane + 64 * c] = p[c];
            p[c] = ph[c] / (1.0f + mr * xk[c] * xk[c] * ph[c]);
        }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const float4 e = make_float4(xa[c], xk[c], xq[c], kap[c]);
        chanw[lane + 64 * c] = e;
        if (rec_chan) rec_chan[lane + 64 * c] = e;
    }
    wave_lds_sync();
    if (stash_tok) {
#pragma unroll
        for (int m = 0; m < RPT; m += SG) stash_tok[snap_idx<RPT>(tid, m)] = snap_pack<RPT>(S, m);
    }
    float Ak[NC] = {};
    float kr[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const float4 c4 = chanw[rg + 8 * m];
        kr[m] = c4.w;
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            S[m][j] *= c4.x;
            Ak[j] += S[m][j] * c4.y;
        }
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) Ak[j] = rowgroup_sum(Ak[j]);
#pragma unroll
    for (int m = 0; m < RPT; ++m)
#pragma unroll
        for (int j = 0; j < NC; ++j) S[m][j] += kr[m] * (xv[j] - Ak[j]);
    wave_lds_sync();  // chanw is rewritten by the next token
}

// In-place halving reduce-scatter over the 8 column lanes of a row
// group: on entry every lane holds N values; on exit lane cq holds, in
// vals[0 .. N/8), the sums over the 8 lanes of flat entries
// [cq * N / 8, (cq + 1) * N / 8).  Step s pairs each lane with one whose
// bit 2 - s differs (7 - cq, then cq ^ 2, then cq ^ 1); each keeps the half
// its own bit selects and receives the partner's copy of that half.
// The halves are chosen with a per-lane bit mask (one bitfield insert per
// value) rather than a compare-and-select, which kept a lane mask in scalar
// registers per select and spilled them.
__device__ __forceinline__ float pick(uint32_t mask, float if_set, float if_clear) {
    // (mask & if_set) | (~mask & if_clear) as one bitfield insert; written
    // out, the compiler emits an and plus an and-or per value
    float r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(mask), "v"(if_set), "v"(if_clear));
    return r;
}

template <int N>
__device__ __forceinline__ void rowsum_scatter(float (&vals)[N], int cq) {
#pragma unroll
    for (int step = 0; step < 3; ++step) {
        const int half = N >> (step + 1);
        const uint32_t hi = 0u - uint32_t((cq >> (2 - step)) & 1);  // all ones when bit X of cq is set
#pragma unroll
        for (int f = 0; f < half; ++f) {
            const float keep = pick(hi, vals[f + half], vals[f]);
            const float send = pick(hi, vals[f], vals[f + half]);
            const float recv = step == 0 ? dpp<DPP_HALF_MIRROR>(send) : step == 1 ? dpp<DPP_XOR2>(send) : dpp<DPP_XOR1>(send);
            vals[f] = keep + recv;
        }
    }
}

constexpr int TILE = 64;  // value columns per memory-adjoint workgroup

// Memory adjoint of one (batch, head) pair over TILE value columns: the
// checkpoint sweep, and per segment the re-run with the stash and the
// reverse walk.  Each token's four per-row sums of the tile (dq, d_kappa,
// dk_mem, dalpha_mem) go to the workspace for the uncertainty kernel; tile 0
// also stores p_{t-1} of every token there.
// GR (diagonal only): grouped observation noise, one r and one uncertainty
// state per tile; the tile's chain uses its group's r and p.
template <int DK, int DV, int VAR, typename Tin, bool GR = false>
__global__ void __launch_bounds__(TILE / WCOLS * 64) kdn_backward_mem_kernel(BwdArgs A) {
    constexpr int NTILE = DV / TILE;
    constexpr int NW = TILE / WCOLS;  // memory waves
    constexpr int CPL = DK / 64;      // channels per lane
    constexpr int RPT = DK / 8;       // memory rows per lane
    constexpr int NT = NW * 64;       // threads
    constexpr bool ISO = VAR != 0;
    static_assert(DK % 64 == 0 && DV % TILE == 0 && NW >= 4 && SEG % PF == 0, "unsupported tile");
    static_assert(!GR || VAR == 0, "grouped noise is a diagonal form");

    __shared__ BwdSmem<DK, TILE> sm;

    const int nunit = A.B * A.H;
    // this round's pairs slot0 .. slot0 + nslot - 1, pair slot0 + s in workspace slot s
    // (wslot; not the LDS ring's slot of the reverse walk below)
    const int nslot = A.nslot ? A.nslot : nunit;
    const int tile = int(blockIdx.x) / nslot;  // the tiles of one head are nslot blocks apart
    const int wslot = int(blockIdx.x) % nslot;
    const int unit = A.slot0 + wslot;
    if (unit >= nunit) return;
    if (A.only_flagged && !A.only_flagged[unit]) return;  // the chunked adjoint took this pair
    const int h = unit % A.H;
    const size_t b = size_t(unit / A.H);
    const int T = A.T;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int tid = threadIdx.x;
    const int cq = lane & 7;
    const int rg = lane >> 3;
    const int col = tile * TILE + wave * WCOLS + cq * NC;
    const int nseg = (T + SEG - 1) / SEG;
    const float mu = A.mu;

    float* ckS = A.work + (size_t(wslot) * NTILE + tile) * unit_floats(T, DK, TILE);
    float* ckP = ckS + size_t(nseg) * DK * TILE;
    // memory snapshots as float4 (m, m + 1) row pairs, see snap_idx
    float4* stash = reinterpret_cast<float4*>(ckP + size_t(nseg) * NW * DK);
    float4* ckS4 = reinterpret_cast<float4*>(ckS);
    constexpr int SNAP = NT * (RPT / SG);  // float4 per snapshot
    float* partial = A.work + size_t(nslot) * NTILE * unit_floats(T, DK, TILE);  // [wslot][T][NTILE][4][DK]
    float* pbuf = partial + size_t(nslot) * T * NTILE * 4 * DK;                    // [wslot][T][NTILE][DK]
    const size_t sbase = size_t(unit) * DK * DV;
    const auto tokidx = [&](int t) { return (b * size_t(T) + size_t(t)) * size_t(A.H) + size_t(h); };

    // ---- forward sweep: checkpoints of (S, p) at every segment start ----
    float S[RPT][NC];
    float p[CPL];
    float pb = 0.f;
    {
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + 8 * m;
#pragma unroll
            for (int j = 0; j < NC; ++j) S[m][j] = A.S0 ? A.S0[sbase + size_t(i) * DV + col + j] : 0.f;
        }
        if (ISO) {
            pb = A.p0 ? A.p0[unit] : A.c0[h];
        } else {
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                p[c] = A.p0 ? A.p0[(GR ? size_t(unit) * NTILE + tile : size_t(unit)) * DK + lane + 64 * c] : A.c0[h];
        }
        for (int seg = 0; seg < nseg; ++seg) {
            float4* ck = ckS4 + size_t(seg) * SNAP;
#pragma unroll
            for (int m = 0; m < RPT; m += SG) ck[snap_idx<RPT>(tid, m)] = snap_pack<RPT>(S, m);
            float* cp = ckP + (size_t(seg) * NW + wave) * DK;
            if (ISO) {
                if (lane == 0) cp[0] = pb;
            } else {
#pragma unroll
                for (int c = 0; c < CPL; ++c) cp[lane + 64 * c] = p[c];
            }
            if (seg == nseg - 1) break;  // the last segment's tokens are re-run below
            // a ring of PF token buffers used in turn: token t + PF - 1 is issued
            // before token t's arithmetic, and no register copy waits for a load
            const int s0 = seg * SEG;
            const auto ld = [&](TokIn<DK, VAR, Tin>& x, int t) {
                load_tok<DK, VAR, Tin, GR>(x, A, tokidx(min(t, T - 1)), lane, col, DV, NTILE, tile);
            };
            const auto run = [&](const TokIn<DK, VAR, Tin>& x) {
                fwd_token<DK, TILE, VAR, Tin>(x, S, p, pb, mu, sm.chan[wave], nullptr, nullptr, nullptr, lane, rg,
                                              tid);
            };
            TokIn<DK, VAR, Tin> x0, x1, x2, x3;
            ld(x0, s0);
            ld(x1, s0 + 1);
            ld(x2, s0 + 2);
            for (int t = s0; t < s0 + SEG; t += PF) {
                ld(x3, t + 3);
                run(x0);
                ld(x0, t + 4);
                run(x1);
                ld(x1, t + 5);
                run(x2);
                ld(x2, t + 6);
                run(x3);
            }
        }
    }

    // ---- reverse sweep, segment by segment ----
    float dS[RPT][NC];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + 8 * m;
#pragma unroll
        for (int j = 0; j < NC; ++j) dS[m][j] = A.dS_T ? A.dS_T[sbase + size_t(i) * DV + col + j] : 0.f;
    }
    const Tin* vin = static_cast<const Tin*>(A.v);
    const Tin* g_src = A.dO ? static_cast<const Tin*>(A.dO) : vin;
    const float g_scale = A.dO ? 1.0f : 0.0f;

    for (int seg = nseg - 1; seg >= 0; --seg) {
        const int t0 = seg * SEG;
        const int n = min(SEG, T - t0);
        {
            // re-run the segment from its checkpoint, recording what the reverse sweep needs
            const float4* ck = ckS4 + size_t(seg) * SNAP;
#pragma unroll
            for (int m = 0; m < RPT; m += SG) snap_unpack<RPT>(S, m, ck[snap_idx<RPT>(tid, m)]);
            const float* cp = ckP + (size_t(seg) * NW + wave) * DK;
            if (ISO) {
                pb = cp[0];
            } else {
#pragma unroll
                for (int c = 0; c < CPL; ++c) p[c] = cp[lane + 64 * c];
            }
            const bool rec = wave == 0;
            const bool rec_p = rec && (GR || tile == 0);  // p_{t-1} of each group
            const auto run = [&](const TokIn<DK, VAR, Tin>& x, int tt) {
                fwd_token<DK, TILE, VAR, Tin>(x, S, p, pb, mu, sm.chan[wave], rec ? sm.seg_chan[tt] : nullptr,
                                              rec_p ? pbuf + ((size_t(wslot) * T + t0 + tt) * NTILE + tile) * DK : nullptr,
                                              stash + size_t(tt) * SNAP, lane, rg, tid);
            };
            const auto ld = [&](TokIn<DK, VAR, Tin>& x, int tt) {
                load_tok<DK, VAR, Tin, GR>(x, A, tokidx(t0 + min(tt, n - 1)), lane, col, DV, NTILE, tile);
            };
            TokIn<DK, VAR, Tin> x0, x1, x2, x3;
            ld(x0, 0);
            ld(x1, 1);
            ld(x2, 2);
            for (int tt = 0; tt < n; tt += PF) {  // loads are always issued (clamped)
                ld(x3, tt + 3);
                run(x0, tt);
                ld(x0, tt + 4);
                if (tt + 1 < n) run(x1, tt + 1);
                ld(x1, tt + 5);
                if (tt + 2 < n) run(x2, tt + 2);
                ld(x2, tt + 6);
                if (tt + 3 < n) run(x3, tt + 3);
            }
        }
        block_lds_sync();

        // PF - 1 tokens ahead, in a ring of PF buffers: S_{t-1}, dO_t, v_t
        struct RevIn {
            float Sp[RPT][NC];
            Tin g[NC], v[NC];
        };
        const auto load_rev = [&](RevIn& r, int tt) {
            const size_t tok = tokidx(t0 + tt);
            const float4* sn = stash + size_t(tt) * SNAP;
#pragma unroll
            for (int m = 0; m < RPT; m += SG) snap_unpack<RPT>(r.Sp, m, sn[snap_idx<RPT>(tid, m)]);
#pragma unroll
            for (int j = 0; j < NC; ++j) {
                // unconditional load (a branch here makes the compiler wait for
                // the prefetch at once): without dO, read v and scale by zero
                r.g[j] = g_src[tok * DV + col + j];
                r.v[j] = vin[tok * DV + col + j];
            }
        };

        // iteration it: token t0 + n - 1 - it; wave w < 4 first writes the
        // tile's sum of quantity w for the token of the iteration before
        const auto iter = [&](int it, const RevIn& cur, RevIn& ahead) {
            if (it >= 1 && wave < 4) {
                const int slot = (it - 1) & 1;
                float* dst = partial + ((size_t(wslot) * T + t0 + n - it) * NTILE + tile) * 4 * DK + size_t(wave) * DK;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int i = lane + 64 * c;
                    float acc = 0.f;
#pragma unroll
                    for (int w = 0; w < NW; ++w) acc += sm.part[slot][wave][w][i];
                    dst[i] = acc;
                }
            }
            if (it < n) {
                const int tt = n - 1 - it;
                const size_t tok = tokidx(t0 + tt);
                const int slot = it & 1;
                const float (&Sp)[RPT][NC] = cur.Sp;  // S_{t-1}
                float g[NC], vv[NC];                   // dO_t, v_t
#pragma unroll
                for (int j = 0; j < NC; ++j) {
                    g[j] = g_scale * to_f32(cur.g[j]);
                    vv[j] = to_f32(cur.v[j]);
                }
                load_rev(ahead, max(tt - (PF - 1), 0));
                const float4* crow = sm.seg_chan[tt];
                // innovation delta = v - S_hat^T k, with S_hat = diag(alpha) S_{t-1};
                // readout cotangent into dS, then d_delta = dS^T kappa
                // the row operands are read from LDS once per token and kept for
                // the three passes (re-reading them in each pass made the LDS
                // return path the limit: 8 waves x 16 rows x 16 B per pass)
                float ra[RPT], rk[RPT], rkap[RPT];
                float Ak[NC] = {}, Ek[NC] = {};
#pragma unroll
                for (int m = 0; m < RPT; ++m) {
                    const float4 c4 = crow[rg + 8 * m];  // (alpha, k, q, kappa) of row rg + 8m
                    ra[m] = c4.x;
                    rk[m] = c4.y;
                    rkap[m] = c4.w;
#pragma unroll
                    for (int j = 0; j < NC; ++j) {
                        Ak[j] += c4.x * Sp[m][j] * c4.y;
                        dS[m][j] += c4.z * g[j];
                        Ek[j] += dS[m][j] * c4.w;
                    }
                }
#pragma unroll
                for (int j = 0; j < NC; ++j) {
                    Ak[j] = rowgroup_sum(Ak[j]);
                    Ek[j] = rowgroup_sum(Ek[j]);
                }
                float dl[NC];
#pragma unroll
                for (int j = 0; j < NC; ++j) dl[j] = vv[j] - Ak[j];
                if (rg == 0) {
#pragma unroll
                    for (int j = 0; j < NC; ++j) A.dv_[tok * DV + col + j] = Ek[j];
                }
                // per-row partial sums over the lane's columns, two quantities
                // at a time: [0] dq = S' dO, [1] d_kappa = dS delta, then
                // [2] dk_mem = -S_hat d_delta, [3] dalpha_mem = sum S_{t-1} (.) dS_hat
                // (and dS <- diag(alpha) dS_hat); after each reduce-scatter lane cq
                // holds quantity cq / 4 of the pair for rows 4 (cq & 3) + e
                const int qh = cq >> 2;
                float vals[2 * RPT];
#pragma unroll
                for (int m = 0; m < RPT; ++m) {
                    float pq = 0.f, pk = 0.f;
#pragma unroll
                    for (int j = 0; j < NC; ++j) {
                        pq += (ra[m] * Sp[m][j] + rkap[m] * dl[j]) * g[j];
                        pk += dS[m][j] * dl[j];
                    }
                    vals[m] = pq;
                    vals[RPT + m] = pk;
                }
                rowsum_scatter<2 * RPT>(vals, cq);
#pragma unroll
                for (int e = 0; e < RPT / 4; ++e)
                    sm.part[slot][qh][wave][rg + 8 * ((cq & 3) * (RPT / 4) + e)] = vals[e];
#pragma unroll
                for (int m = 0; m < RPT; ++m) {
                    float pks = 0.f, pa = 0.f;
#pragma unroll
                    for (int j = 0; j < NC; ++j) {
                        pks -= ra[m] * Sp[m][j] * Ek[j];
                        const float dsh = dS[m][j] - rk[m] * Ek[j];
                        pa += Sp[m][j] * dsh;
                        dS[m][j] = ra[m] * dsh;
                    }
                    vals[m] = pks;
                    vals[RPT + m] = pa;
                }
                rowsum_scatter<2 * RPT>(vals, cq);
#pragma unroll
                for (int e = 0; e < RPT / 4; ++e)
                    sm.part[slot][2 + qh][wave][rg + 8 * ((cq & 3) * (RPT / 4) + e)] = vals[e];
            }
            block_lds_sync();
        };
        RevIn r0, r1, r2, r3;
        load_rev(r0, n - 1);
        load_rev(r1, max(n - 2, 0));
        load_rev(r2, max(n - 3, 0));
        for (int it = 0; it <= n; it += PF) {
            iter(it, r0, r3);
            if (it + 1 <= n) iter(it + 1, r1, r0);
            if (it + 2 <= n) iter(it + 2, r2, r1);
            if (it + 3 <= n) iter(it + 3, r3, r2);
        }
    }

#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + 8 * m;
#pragma unroll
        for (int j = 0; j < NC; ++j) A.dS0[sbase + size_t(i) * DV + col + j] = dS[m][j];
    }
}

// Uncertainty adjoint of one (batch, head) pair, one wave (lane owns channels
// lane and lane + 64), backwards over the tokens: sums the memory kernel's
// per-tile row sums, writes dq, dk, dalpha, domega, dr and carries dp.
template <int DK, int DV, int VAR, typename Tin>
__global__ void __launch_bounds__(64) kdn_backward_unc_kernel(BwdArgs A) {
    constexpr int NTILE = DV / TILE;
    constexpr int CPL = DK / 64;
    constexpr bool ISO = VAR != 0;
    const int nunit = A.B * A.H;
    const int nslot = A.nslot ? A.nslot : nunit;
    const int wslot = int(blockIdx.x);
    const int unit = A.slot0 + wslot;
    if (unit >= nunit) return;
    if (A.only_flagged && !A.only_flagged[unit]) return;  // the chunked path's adjoint took this pair
    const int h = unit % A.H;
    const size_t b = size_t(unit / A.H);
    const int T = A.T;
    const int lane = threadIdx.x;
    const float mu = A.mu;
    const float* partial = A.work + size_t(nslot) * NTILE * unit_floats(T, DK, TILE);
    const float* pbuf = partial + size_t(nslot) * T * NTILE * 4 * DK;
    const Tin* kin = static_cast<const Tin*>(A.k);
    const Tin* ain = static_cast<const Tin*>(A.alpha);
    const Tin* omg = static_cast<const Tin*>(A.omega);
    const Tin* rr = static_cast<const Tin*>(A.r);
    const auto tokidx = [&](int t) { return (b * size_t(T) + size_t(t)) * size_t(A.H) + size_t(h); };

    float dp[CPL];
    float db = 0.f;
    if (ISO) {
        db = A.dp_T ? A.dp_T[unit] : 0.f;
    } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) dp[c] = A.dp_T ? A.dp_T[size_t(unit) * DK + lane + 64 * c] : 0.f;
    }

    // PF - 1 tokens ahead, in a ring of PF buffers: the tile sums, p_{t-1}
    // and the token's alpha, k, omega, r
    struct UncIn {
        float q[CPL], k[CPL], ks[CPL], a[CPL], pp[CPL];
        Tin al[CPL], kk[CPL], w[CPL], r;
    };
    const auto load = [&](UncIn& u, int t) {
        const size_t tok = tokidx(t);
        const float* src = partial + (size_t(wslot) * T + t) * NTILE * 4 * DK;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int i = lane + 64 * c;
            u.q[c] = u.k[c] = u.ks[c] = u.a[c] = 0.f;
#pragma unroll
            for (int tl = 0; tl < NTILE; ++tl) {
                u.q[c] += src[(tl * 4 + 0) * DK + i];
                u.k[c] += src[(tl * 4 + 1) * DK + i];
                u.ks[c] += src[(tl * 4 + 2) * DK + i];
                u.a[c] += src[(tl * 4 + 3) * DK + i];
            }
            u.al[c] = VAR == 1 ? ain[tok] : ain[tok * DK + i];
            u.kk[c] = kin[tok * DK + i];
            u.pp[c] = ISO ? pbuf[(size_t(wslot) * T + t) * NTILE * DK] : pbuf[(size_t(wslot) * T + t) * NTILE * DK + i];
            u.w[c] = VAR == 0 ? omg[tok * DK + i] : omg[tok];
        }
        u.r = rr[tok];
    };
    const auto step = [&](int t, const UncIn& u, UncIn& ahead) {
        const size_t tok = tokidx(t);
        float al[CPL], kk[CPL], pp[CPL], gq[CPL], gk[CPL], gks[CPL], ga[CPL], wc[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            al[c] = to_f32(u.al[c]); kk[c] = to_f32(u.kk[c]); pp[c] = u.pp[c]; wc[c] = to_f32(u.w[c]);
            gq[c] = u.q[c]; gk[c] = u.k[c]; gks[c] = u.ks[c]; ga[c] = u.a[c];
        }
        const float rt = to_f32(u.r);
        load(ahead, max(t - (PF - 1), 0));
#pragma unroll
        for (int c = 0; c < CPL; ++c) A.dq[tok * DK + lane + 64 * c] = gq[c];
                if (!ISO) {
                    // gain kappa = p_hat k / d, d = r + sum p_hat k^2; posterior
                    // p' = p_hat / (1 + u p_hat), u = (mu / r) k^2; predict
                    // p_hat = alpha^2 p + omega
                    float ph[CPL];
                    float s = 0.f;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        ph[c] = al[c] * al[c] * pp[c] + wc[c];
                        s += ph[c] * kk[c] * kk[c];
                    }
                    s = wave_sum(s);
                    const float d = rt + s;
                    const float inv = 1.0f / d;
                    float kd = 0.f;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) kd += gk[c] * ph[c] * kk[c];
                    const float dd = -wave_sum(kd) * inv * inv;
                    const float mr = mu / rt;
                    float drr = 0.f;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const int i = lane + 64 * c;
                        const float k2 = kk[c] * kk[c];
                        const float den = 1.0f + mr * k2 * ph[c];
                        const float pn = ph[c] / den;
                        const float du = -dp[c] * pn * pn;
                        const float dph = dp[c] / (den * den) + gk[c] * kk[c] * inv + dd * k2;
                        drr -= du * mr * k2 / rt;
                        A.dk_[tok * DK + i] = gks[c] + gk[c] * ph[c] * inv + 2.0f * dd * ph[c] * kk[c] +
                                              2.0f * du * mr * kk[c];
                        A.dalpha[tok * DK + i] = ga[c] + 2.0f * dph * al[c] * pp[c];
                        A.domega[tok * DK + i] = dph;
                        dp[c] = dph * al[c] * al[c];
                    }
                    drr = wave_sum(drr);
                    if (lane == 0) A.dr[tok] = dd + drr;
                } else {
                    // scalar gain beta = b_hat / (r + b_hat n), n = |k|^2; posterior
                    // b' = b_hat / (1 + c n b_hat), c = mu / (d_k r); predict
                    // b_hat = a b + omega / d_k, a = alpha^2 or mean_i alpha_i^2
                    const float bprev = pp[0];
                    const float w = wc[0];
                    float a2 = 0.f, nn = 0.f, kb = 0.f;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        a2 += al[c] * al[c];
                        nn += kk[c] * kk[c];
                        kb += gk[c] * kk[c];
                    }
                    a2 = VAR == 2 ? wave_sum(a2) * (1.0f / float(DK)) : al[0] * al[0];
                    nn = wave_sum(nn);
                    const float dbeta = wave_sum(kb);
                    const float bh = a2 * bprev + w * (1.0f / float(DK));
                    const float dg = rt + bh * nn;
                    const float beta = bh / dg;
                    const float cc = mu / (float(DK) * rt);
                    const float dpn = 1.0f + cc * nn * bh;
                    const float bt = bh / dpn;
                    const float idg2 = 1.0f / (dg * dg);
                    const float dbh = dbeta * rt * idg2 + db / (dpn * dpn);
                    const float dn = -dbeta * bh * bh * idg2 - db * bt * bt * cc;
                    const float dR = -dbeta * bh * idg2 + db * bt * bt * cc * nn / rt;
                    float gas = 0.f;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const int i = lane + 64 * c;
                        A.dk_[tok * DK + i] = gks[c] + beta * gk[c] + 2.0f * dn * kk[c];
                        if (VAR == 2) A.dalpha[tok * DK + i] = ga[c] + dbh * bprev * 2.0f * al[c] * (1.0f / float(DK));
                        gas += ga[c];
                    }
                    if (VAR == 1) gas = wave_sum(gas);
                    if (lane == 0) {
                        if (VAR == 1) A.dalpha[tok] = gas + 2.0f * dbh * al[0] * bprev;
                        A.domega[tok] = dbh * (1.0f / float(DK));
                        A.dr[tok] = dR;
                    }
                    db = dbh * a2;
                }
    };
    UncIn u0, u1, u2, u3;
    if (T > 0) {
        load(u0, T - 1);
        load(u1, max(T - 2, 0));
        load(u2, max(T - 3, 0));
    }
    for (int t = T - 1; t >= 0; t -= PF) {
        step(t, u0, u3);
        if (t - 1 >= 0) step(t - 1, u1, u0);
        if (t - 2 >= 0) step(t - 2, u2, u1);
        if (t - 3 >= 0) step(t - 3, u3, u2);
    }


    if (ISO) {
        if (lane == 0) A.dp0[unit] = db;
    } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) A.dp0[size_t(unit) * DK + lane + 64 * c] = dp[c];
    }
}

// Uncertainty adjoint of the grouped-noise form, one wave per (batch, head):
// per token and group, the diagonal uncertainty adjoint with the group's r,
// p_{t-1}, carried dp and its tile's row sums; the gradients of the shared
// k, alpha, omega are summed over the groups, dr and dp0 are per group.
template <int DK, int DV, typename Tin>
__global__ void __launch_bounds__(64) kdn_backward_unc_grouped_kernel(BwdArgs A) {
    constexpr int G = DV / TILE;
    constexpr int CPL = DK / 64;
    const int nunit = A.B * A.H;
    const int nslot = A.nslot ? A.nslot : nunit;
    const int wslot = int(blockIdx.x);
    const int unit = A.slot0 + wslot;
    if (unit >= nunit) return;
    const int h = unit % A.H;
    const size_t b = size_t(unit / A.H);
    const int T = A.T;
    const int lane = threadIdx.x;
    const float mu = A.mu;
    const float* partial = A.work + size_t(nslot) * G * unit_floats(T, DK, TILE);
    const float* pbuf = partial + size_t(nslot) * T * G * 4 * DK;
    const Tin* kin = static_cast<const Tin*>(A.k);
    const Tin* ain = static_cast<const Tin*>(A.alpha);
    const Tin* omg = static_cast<const Tin*>(A.omega);
    const Tin* rr = static_cast<const Tin*>(A.r);
    const auto tokidx = [&](int t) { return (b * size_t(T) + size_t(t)) * size_t(A.H) + size_t(h); };

    float dp[G][CPL];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            dp[g][c] = A.dp_T ? A.dp_T[(size_t(unit) * G + g) * DK + lane + 64 * c] : 0.f;

    struct UncG {
        float q[CPL], k[G][CPL], ks[G][CPL], a[G][CPL], pp[G][CPL];
        Tin al[CPL], kk[CPL], w[CPL], r[G];
    };
    const auto load = [&](UncG& u, int t) {
        const size_t tok = tokidx(t);
        const float* src = partial + (size_t(wslot) * T + t) * G * 4 * DK;
        const float* ps = pbuf + (size_t(wslot) * T + t) * G * DK;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int i = lane + 64 * c;
            u.q[c] = 0.f;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                u.q[c] += src[(g * 4 + 0) * DK + i];
                u.k[g][c] = src[(g * 4 + 1) * DK + i];
                u.ks[g][c] = src[(g * 4 + 2) * DK + i];
                u.a[g][c] = src[(g * 4 + 3) * DK + i];
                u.pp[g][c] = ps[g * DK + i];
            }
            u.al[c] = ain[tok * DK + i];
            u.kk[c] = kin[tok * DK + i];
            u.w[c] = omg[tok * DK + i];
        }
#pragma unroll
        for (int g = 0; g < G; ++g) u.r[g] = rr[tok * G + g];
    };
    const auto step = [&](int t, const UncG& u, UncG& ahead) {
        const size_t tok = tokidx(t);
        float al[CPL], kk[CPL], wc[CPL], dkacc[CPL], daacc[CPL], dwacc[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            al[c] = to_f32(u.al[c]);
            kk[c] = to_f32(u.kk[c]);
            wc[c] = to_f32(u.w[c]);
            dkacc[c] = daacc[c] = dwacc[c] = 0.f;
            A.dq[tok * DK + lane + 64 * c] = u.q[c];
        }
        float rg[G];
#pragma unroll
        for (int g = 0; g < G; ++g) rg[g] = to_f32(u.r[g]);
        load(ahead, max(t - (PF - 1), 0));
#pragma unroll
        for (int g = 0; g < G; ++g) {
            // the diagonal uncertainty adjoint of group g (gain, posterior, predict)
            const float rt = rg[g];
            float ph[CPL];
            float s = 0.f, kd = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                ph[c] = al[c] * al[c] * u.pp[g][c] + wc[c];
                s += ph[c] * kk[c] * kk[c];
                kd += u.k[g][c] * ph[c] * kk[c];
            }
            s = wave_sum(s);
            const float d = rt + s;
            const float inv = 1.0f / d;
            const float dd = -wave_sum(kd) * inv * inv;
            const float mr = mu / rt;
            float drr = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const float k2 = kk[c] * kk[c];
                const float den = 1.0f + mr * k2 * ph[c];
                const float pn = ph[c] / den;
                const float du = -dp[g][c] * pn * pn;
                const float dph = dp[g][c] / (den * den) + u.k[g][c] * kk[c] * inv + dd * k2;
                drr -= du * mr * k2 / rt;
                dkacc[c] += u.ks[g][c] + u.k[g][c] * ph[c] * inv + 2.0f * dd * ph[c] * kk[c] + 2.0f * du * mr * kk[c];
                daacc[c] += u.a[g][c] + 2.0f * dph * al[c] * u.pp[g][c];
                dwacc[c] += dph;
                dp[g][c] = dph * al[c] * al[c];
            }
            drr = wave_sum(drr);
            if (lane == 0) A.dr[tok * G + g] = dd + drr;
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int i = lane + 64 * c;
            A.dk_[tok * DK + i] = dkacc[c];
            A.dalpha[tok * DK + i] = daacc[c];
            A.domega[tok * DK + i] = dwacc[c];
        }
    };
    UncG u0, u1, u2, u3;
    if (T > 0) {
        load(u0, T - 1);
        load(u1, max(T - 2, 0));
        load(u2, max(T - 3, 0));
    }
    for (int t = T - 1; t >= 0; t -= PF) {
        step(t, u0, u3);
        if (t - 1 >= 0) step(t - 1, u1, u0);
        if (t - 2 >= 0) step(t - 2, u2, u1);
        if (t - 3 >= 0) step(t - 3, u3, u2);
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < CPL; ++c) A.dp0[(size_t(unit) * G + g) * DK + lane + 64 * c] = dp[g][c];
}

// dc0[h] = sum over the batch and the channels of dp0 (the c0 gradient when
// p_0 = c0[h] on every channel): one wave per head, each lane summing a fixed
// strided subset, then a fixed-order wave sum
__global__ void __launch_bounds__(64) kdn_dc0_kernel(const float* __restrict__ dp0, float* __restrict__ dc0,
                                                     int B, int H, int pd) {
    const int h = int(blockIdx.x);
    const int lane = int(threadIdx.x);
    const long n = long(B) * pd;
    float acc = 0.f;
    for (long e = lane; e < n; e += 64) acc += dp0[(size_t(e / pd) * H + h) * pd + size_t(e % pd)];
    acc = wave_sum(acc);
    if (lane == 0) dc0[h] = acc;
}

// The token path in rounds of as many pairs as the workspace from a.work
// holds (every pair at once with backward_workspace_bytes()).
template <typename F>
hipError_t in_rounds(const BwdArgs& a, F&& launch) {
    const int units = a.B * a.H;
    const size_t per = token_pair_bytes(a.T, a.dk, a.dv);
    // (T = 0 touches no workspace: the cotangents pass straight through)
    const int k = a.T == 0 ? units : int(std::min<size_t>(size_t(units), a.work_bytes / per));
    if (k < 1) return hipErrorInvalidValue;
    BwdArgs r = a;
    r.nslot = k;
    for (int s0 = 0; s0 < units; s0 += k) {
        r.slot0 = s0;
        const hipError_t e = launch(r);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DK, int DV, int VAR, typename Tin>
hipError_t launch_t(const BwdArgs& a, hipStream_t stream) {
    return in_rounds(a, [&](const BwdArgs& r) {
        const unsigned n = unsigned(r.nslot);
        hipLaunchKernelGGL((kdn_backward_mem_kernel<DK, DV, VAR, Tin>), dim3(n * (DV / TILE)), dim3(TILE / WCOLS * 64), 0,
                           stream, r);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((kdn_backward_unc_kernel<DK, DV, VAR, Tin>), dim3(n), dim3(64), 0, stream, r);
        return hipGetLastError();
    });
}

template <int DK, int DV, int VAR>
hipError_t launch_dtype(const BwdArgs& a, hipStream_t s) {
    return a.dtype == 1 ? launch_t<DK, DV, VAR, bf16_t>(a, s) : launch_t<DK, DV, VAR, float>(a, s);
}

template <int DK, int DV, typename Tin>
hipError_t launch_grouped_t(const BwdArgs& a, hipStream_t stream) {
    return in_rounds(a, [&](const BwdArgs& r) {
        const unsigned n = unsigned(r.nslot);
        hipLaunchKernelGGL((kdn_backward_mem_kernel<DK, DV, 0, Tin, true>), dim3(n * (DV / TILE)),
                           dim3(TILE / WCOLS * 64), 0, stream, r);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((kdn_backward_unc_grouped_kernel<DK, DV, Tin>), dim3(n), dim3(64), 0, stream, r);
        return hipGetLastError();
    });
}

// The chunked path for the diagonal bf16 form, in two parts, on the
// workspace layout of ChunkWs.  main: the chunked forward's checkpoint sweep
// (chunk-start states in bf16 and uncertainties, one range flag per (batch,
// head) pair), then per slab of tokens, from the last, the chunked memory
// adjoint (kdn_backward_chunk.hip) and the uncertainty adjoint of the
// unflagged pairs, carrying dS and dp from slab to slab; then dr.
// fallback: the token path with fb's arguments (a itself, or for the gated
// layer its fp32 copies of the gated values) for the flagged pairs, in
// rounds over the workspace after the flags.
ChunkWs chunk_layout(const BwdArgs& a) {
    ChunkWs w{};
    chunk_workspace(a.B, a.T, a.H, a.dk, a.dv, a.work, a.work_bytes, &w);
    return w;
}

hipError_t chunked_main(const BwdArgs& a, hipStream_t s) {
    ChunkWs w{};
    if (!chunk_workspace(a.B, a.T, a.H, a.dk, a.dv, a.work, a.work_bytes, &w)) return hipErrorInvalidValue;
    FwdArgs f{a.q, a.k, a.v, a.alpha, a.omega, a.r, a.c0, a.mu, 0, 1, a.B, a.T, a.H, a.dk, a.dv,
              a.S0, a.p0, nullptr, nullptr, nullptr};
    f.gates = a.gates;
    hipError_t e = launch_chunked_checkpoints(f, w.cks, w.ckp, w.flag, s);
    for (int j = w.nslab - 1; j >= 0 && e == hipSuccess; --j) {
        e = launch_backward_chunk(a, w, j, s);
        if (e == hipSuccess) e = launch_backward_unc_chunk(a, w, j, s);
    }
    return e != hipSuccess ? e : launch_backward_dr(a, w, s);
}

template <int DK, int DV>
hipError_t chunked_fallback(const BwdArgs& a, const BwdArgs& fb, hipStream_t s) {
    const ChunkWs w = chunk_layout(a);
    BwdArgs r = fb;
    r.only_flagged = w.flag;
    r.work = reinterpret_cast<float*>(w.rest);
    r.work_bytes = w.rest_bytes;
    r.gates = false;
    return fb.dtype == 1 ? launch_t<DK, DV, 0, bf16_t>(r, s) : launch_t<DK, DV, 0, float>(r, s);
}

template <int DK, int DV>
hipError_t launch_chunked_path(const BwdArgs& a, const BwdArgs& fb, hipStream_t s) {
    const hipError_t e = chunked_main(a, s);
    return e != hipSuccess ? e : chunked_fallback<DK, DV>(a, fb, s);
}

bool chunk_path(const BwdArgs& a) {
    const auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    const bool aligned = al16(a.q) && al16(a.k) && al16(a.v) && al16(a.alpha) && al16(a.omega) && al16(a.dO);
    FwdArgs f{a.q, a.k, a.v, a.alpha, a.omega, a.r, a.c0, a.mu, 0, 1, a.B, a.T, a.H, a.dk, a.dv,
              a.S0, a.p0, nullptr, nullptr, nullptr};
    return a.variant == 0 && a.dtype == 1 && a.T > 0 && aligned && chunked_supports(f);
}

template <int DK, int DV>
hipError_t launch_variant(const BwdArgs& a, hipStream_t s) {
    if (a.variant == 3)  // diagonal with grouped observation noise
        return a.dtype == 1 ? launch_grouped_t<DK, DV, bf16_t>(a, s) : launch_grouped_t<DK, DV, float>(a, s);
    if (a.variant == 2) return launch_dtype<DK, DV, 2>(a, s);
    if (chunk_path(a)) return launch_chunked_path<DK, DV>(a, a, s);
    return a.variant == 1 ? launch_dtype<DK, DV, 1>(a, s) : launch_dtype<DK, DV, 0>(a, s);
}

}  // namespace

size_t token_pair_bytes(int T, int dk, int dv) {
    const size_t ntile = size_t(dv) / TILE;
    // per tile checkpoints and stash; per token the tile sums and p_{t-1} (per tile)
    return (ntile * unit_floats(T, dk, TILE) + size_t(T) * ntile * 5 * dk) * sizeof(float);
}

size_t backward_workspace_bytes(int B, int T, int H, int dk, int dv) {
    if (long(B) * H == 0 || T == 0) return 0;
    // every pair on the token path at once, plus the chunked path's range
    // flags (its layout fits in this size: bf16 checkpoints, longer slabs)
    const size_t units = size_t(B) * size_t(H);
    return units * token_pair_bytes(T, dk, dv) + ((units * sizeof(int) + 255) & ~size_t(255));
}

size_t backward_workspace_bytes_for(int variant, int dtype, int B, int T, int H, int dk, int dv) {
    if (long(B) * H == 0 || T == 0) return 0;
    const bool chunked = variant == 0 && dtype == 1 && (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
    if (!chunked) return backward_workspace_bytes(B, T, H, dk, dv);
    // the chunked layout, and room after the flags for one pair on the token
    // path (pairs outside the chunked range, or inputs it cannot take)
    const size_t flags = ((size_t(B) * size_t(H) * sizeof(int)) + 255) & ~size_t(255);
    return std::max(chunk_workspace_min_bytes(B, T, H, dk, dv), flags + token_pair_bytes(T, dk, dv));
}

bool backward_chunked_eligible(const BwdArgs& a) {
    return (a.dk == 128 || a.dk == 64) && (a.dv == 128 || a.dv == 64) && chunk_path(a);
}

int* backward_chunk_flags(const BwdArgs& a) { return chunk_layout(a).flag; }

hipError_t launch_backward_chunked_main(const BwdArgs& a, hipStream_t stream) { return chunked_main(a, stream); }

hipError_t launch_backward_chunked_fallback(const BwdArgs& a, const BwdArgs& fallback, hipStream_t stream) {
    hipError_t e;
    if (a.dk == 128 && a.dv == 128) e = chunked_fallback<128, 128>(a, fallback, stream);
    else if (a.dk == 128 && a.dv == 64) e = chunked_fallback<128, 64>(a, fallback, stream);
    else if (a.dk == 64 && a.dv == 128) e = chunked_fallback<64, 128>(a, fallback, stream);
    else if (a.dk == 64 && a.dv == 64) e = chunked_fallback<64, 64>(a, fallback, stream);
    else return hipErrorNotSupported;
    if (e != hipSuccess || !a.dc0) return e;
    hipLaunchKernelGGL(kdn_dc0_kernel, dim3(unsigned(a.H)), dim3(64), 0, stream, a.dp0, a.dc0, a.B, a.H, a.dk);
    return hipGetLastError();
}

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
    hipError_t e;
    if (a.dk == 128 && a.dv == 128) e = launch_variant<128, 128>(a, stream);
    else if (a.dk == 128 && a.dv == 64) e = launch_variant<128, 64>(a, stream);
    else if (a.dk == 64 && a.dv == 128) e = launch_variant<64, 128>(a, stream);
    else if (a.dk == 64 && a.dv == 64) e = launch_variant<64, 64>(a, stream);
    else return hipErrorNotSupported;
    if (e != hipSuccess || !a.dc0) return e;
    const int pd = a.variant == 0 ? a.dk : a.variant == 3 ? (a.dv / TILE) * a.dk : 1;
    hipLaunchKernelGGL(kdn_dc0_kernel, dim3(unsigned(a.H)), dim3(64), 0, stream, a.dp0, a.dc0, a.B, a.H, pd);
    return hipGetLastError();
}

}  // namespace kdn
