// kdn_iso.hip -- chunkwise forward of the isotropic KDN variant on gfx950,
// with the decay weights applied to Gram matrices of the raw keys.
//
// Method ("Kalman Delta Networks: Uncertainty-aware Associative Memory",
// summary page, method steps 2-5 and the isotropic closing sentence).  Per
// (batch, head), one uncertainty scalar b and scalar decay alpha_t per token:
//   b_hat = alpha^2 b + omega / d_k;  kappa = k b_hat / (r + b_hat |k|^2)
//   S = alpha S + kappa (v - alpha S^T k)^T;  o = S^T q
//   b = b_hat / (1 + (mu / (d_k r)) |k|^2 b_hat)
//
// Chunk form (our derivation from those steps).  With chunks of L = 32 tokens,
// G_t = sum_{u<=t in the chunk} log2 alpha_u, and Dn_t the innovation over its
// gain denominator d_t = r_t + b_hat_t |k_t|^2, the token recurrence inside a
// chunk is exactly
//   M Dn = V - diag(2^G) K S_c,     M_ts = r_t [t = s] + b_hat_s 2^(G_t - G_s) (k_t . k_s)   (s <= t)
//   O    = diag(2^G) Q S_c + P Dn,  P_ts = b_hat_s 2^(G_t - G_s) (q_t . k_s)                   (s <= t)
//   S_{c+1} = 2^(G_L) S_c + K^T diag(w) Dn,   w_s = b_hat_s 2^(G_L - G_s)
// Because the decay is one scalar per token, every decay factor lands on a
// row or a column: the matrix cores take the raw bf16 k and q tiles (the Gram
// matrices K K^T and Q K^T, K S_c, Q S_c, K^T Dn) and the weights are applied
// in fp32 to 32 x 32 matrices and to rows.  Every weight used is
// 2^(non-positive), so the form holds for every 0 < alpha <= 1 with nothing
// to overflow (log2 alpha is floored at -150, below which 2^x is zero in
// fp32 anyway).
//
// The memory is carried as S = Gamma S~ with a scalar Gamma in [2^-64, 1]:
// the chunk's own decay goes into Gamma (and into the row weights of R and
// O and the column weights of the update), so the state needs no per-chunk
// rescale; only when Gamma would fall below 2^-64 is S~ multiplied through.
//
// Workgroup = one (batch, head) pair and 64 value columns (32 when the
// 64-column tiling would leave more than half of the CUs idle), 8 waves, in a
// software pipeline with one workgroup barrier per iteration: at iteration i
//   wave 0  scan of chunk i: the uncertainty scalar's Mobius maps over the
//           chunk's 32 tokens (lane = token) from |k_t|^2 (gated: computed
//           here from the chunk's k tile), composed as 2 x 2 matrix products
//           by an inclusive cross-lane scan on DPP row shifts and a row
//           broadcast; the log-decay prefix sums the same way; per-token
//           weights to LDS
//   wave 1  Gram K K^T of chunk i - 1 (matrix cores), weighted into M's
//           diagonal blocks and -M_10; not gated, tile (1,1) of P of chunk
//           i - 1; k^T of chunk i - 2 for the update
//   wave 2  inverses of M's diagonal blocks of chunk i - 2; not gated, tiles
//           (0,0) and (1,0) of the Gram Q K^T of chunk i - 1, weighted into
//           P = tril(...)
//   wave 3  direct copies of the k and q tiles of chunk i + 2; |k_t|^2 of
//           chunk i + 1 once its tile has landed (not gated); gated, the
//           query norms and P of chunk i - 1 (each SIMD runs one state wave
//           and one of waves 0..3, so the other roles' work is spread so that
//           no SIMD pair carries much more than the others)
//   waves 4..7  state update of chunk i - 3: 16 value columns each, S~ in
//           registers (fp32)
// Everything a wave reads at iteration i was written before the barrier that
// ended iteration i - 1, so the roles overlap and an iteration costs the
// slowest of them.
#include "kdn_device.h"
#include "kdn_gates.h"
#include "kdn_internal.h"

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace kdn {
namespace {

using namespace dev;

constexpr int L = 32;          // tokens per chunk
constexpr int NT = L / 16;     // 16-token tiles per chunk
constexpr int NTHREADS = 512;  // 8 waves
constexpr int PT = L + 8;      // pitch of the bf16 P rows
constexpr int KR = 6;          // ring of k and q tiles: a chunk's tiles live from their copy (two iterations
                               // ahead) to the state's read (three iterations behind)
constexpr float kLogFloor = -150.f;  // log2 alpha below this: 2^x is zero in fp32
constexpr float kFrameMin = 0x1p-64f;  // Gamma is kept at or above this

template <int DK>
struct IsoSmem {
    alignas(16) bf16_t K[KR][L * DK];     // k tiles [t][sw(i)] (direct copies)
    alignas(16) bf16_t Q[KR][L * DK];     // q tiles [t][sw(i)]
    alignas(16) bf16_t KT[2][L * DK];     // k^T [P / 8][i][P % 8] with P = perm32(t): the update's A operand
    alignas(16) bf16_t RV[3][L * 64];     // v tiles of the state waves ([wave][t][16 NCW columns]), ring of three
    alignas(16) float sc[4][6][L];        // per chunk (slot c % 4): r, b_hat, G, row weight of R (2^G Gamma_c;
                                          // gated: times 1/|k_t|), 1/|k_t| (gated), row weight of O (gated)
    alignas(16) float ws[4][L];           // update column weights w_s / (the frame change), per chunk
    alignas(16) float ch[4][4];           // per chunk: the C-input factor of the update (1 = none), Gamma_c
    alignas(16) bf16_t P[3][L * PT];      // tril(P) [t][perm32(s)] (ring of three)
    alignas(16) bf16_t Td[2][NT * 256];   // inverses of M's diagonal blocks [a][t][s]
    alignas(16) bf16_t Mo[3][256];        // -M_10 [t][s]
    alignas(16) float Md[2][NT * 256];    // M's diagonal blocks, column-major [a][s][t]
    alignas(16) float Wi[NT][2][64];      // block-inverse scratch
    alignas(16) float qn[L];              // 1/|q_t| of the Gram-P wave's chunk (gated)
    alignas(16) float kn[2][L];           // |k_t|^2 of the next chunk (slot c & 1), for the scan
};

struct IsoArgs {
    const bf16_t* q;
    const bf16_t* k;
    const bf16_t* v;
    const bf16_t* alpha;
    const bf16_t* omega;
    const bf16_t* r;
    const float* c0;
    float mu;
    int T, H, DV, units;
    const float* S0;
    const float* p0;
    bf16_t* o;
    float* S_T;
    float* p_T;
    const int* cu;
    const int* ord;
    size_t tok0;
};

__device__ __forceinline__ size_t tokidx(const IsoArgs& a, int h, int t) {
    return (a.tok0 + size_t(t)) * size_t(a.H) + size_t(h);
}

// ---------------------------------------------------------------------------
// cross-lane steps on DPP (data moves inside a VALU instruction).  Within
// each 16-lane row, row_shr:d takes lane i - d (lanes below d keep `old`);
// row_bcast:15 with row mask 0b1010 gives rows 1 and 3 lane 15 of the row
// below.  Lanes 0..31 and 32..63 are two copies of the same 32 tokens.
// ---------------------------------------------------------------------------
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ float dpp(float old, float src) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, ROWMASK,
                                                      0xf, false));
}
constexpr int kRowShr = 0x110;     // + shift
constexpr int kRowBcast15 = 0x142;
constexpr int kWaveShr1 = 0x138;

// one level of the inclusive scan of 2 x 2 Mobius matrices (this x earlier,
// renormalised so that m11 = 1) and of the log-decay sums
template <int CTRL, int ROWMASK>
__device__ __forceinline__ void scan_level(float& m00, float& m01, float& m10, float& m11, float& g) {
    const float x00 = dpp<CTRL, ROWMASK>(1.f, m00), x01 = dpp<CTRL, ROWMASK>(0.f, m01);
    const float x10 = dpp<CTRL, ROWMASK>(0.f, m10), x11 = dpp<CTRL, ROWMASK>(1.f, m11);
    const float xg = dpp<CTRL, ROWMASK>(0.f, g);
    const float y00 = fmaf(m00, x00, m01 * x10), y01 = fmaf(m00, x01, m01 * x11);
    const float y10 = fmaf(m10, x00, m11 * x10), y11 = fmaf(m10, x01, m11 * x11);
    const float s = __builtin_amdgcn_rcpf(y11);
    m00 = y00 * s;
    m01 = y01 * s;
    m10 = y10 * s;
    m11 = 1.f;
    g += xg;
}

// ---------------------------------------------------------------------------
// scan wave: lane = token (lanes 32..63 repeat lanes 0..31)
// ---------------------------------------------------------------------------
struct ScanRegs {
    bf16_t al, w, rv;  // alpha, omega, r of token lane & 31
};

__device__ __forceinline__ void scan_load(ScanRegs& X, const IsoArgs& a, int h, int c, int nchunks) {
    c = min(max(c, 0), nchunks - 1);
    const int lane = threadIdx.x & 63;
    const size_t e = tokidx(a, h, min(c * L + (lane & 31), a.T - 1));
    X.al = a.alpha[e];
    X.w = a.omega[e];
    X.rv = a.r[e];
}

// |k_t|^2 of token t = lane & 31 of a k tile (lanes l and l + 32 each sum
// half of the row in fp32, then exchange)
template <int DK>
__device__ __forceinline__ float tile_norm(const bf16_t* K) {
    const int lane = threadIdx.x & 63;
    const int t = lane & 31, half = lane >> 5;
    constexpr int PCS = DK / 16;  // 16-byte pieces per half row
    float n = 0.f;
#pragma unroll
    for (int m = 0; m < PCS; ++m) {
        const u4 x = *reinterpret_cast<const u4*>(K + sw<DK>(t, 8 * (half * PCS + m)));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x0 = bf_lo(x[e]), x1 = bf_hi(x[e]);
            n = fmaf(x0, x0, n);
            n = fmaf(x1, x1, n);
        }
    }
    return n + __shfl_xor(n, 32, 64);
}

template <int DK, bool GATE>
__device__ __forceinline__ void scan_run(const ScanRegs& X, IsoSmem<DK>& sm, int c, float n, float mu,
                                         float& bprev, float& gam, int nvalid) {
    const int lane = threadIdx.x & 63;
    const int t = lane & 31;
    const bool ok = t < nvalid;
    float az = bf1(X.al), wz = bf1(X.w), rz = bf1(X.rv);
    float lg;  // log2 alpha
    float al;
    if (GATE) {
        // alpha = 1 / (1 + e^-z): log2 alpha = -log2(1 + e^-z), exact also where alpha underflows
        const float ez = __builtin_amdgcn_exp2f(-kLog2E * az);
        al = __builtin_amdgcn_rcpf(1.f + ez);
        lg = -__builtin_amdgcn_logf(1.f + ez);
        wz = gate_softplus(wz);
        rz = kGateRMin + gate_softplus(rz);
    } else {
        al = az;
        lg = __builtin_amdgcn_logf(az);
    }
    lg = ok ? fmaxf(lg, kLogFloor) : 0.f;
    al = ok ? al : 1.f;
    const float asq = al * al;
    const float w = ok ? wz * (1.f / float(DK)) : 0.f;
    const float rt = ok ? rz : 1.f;
    // gated: the prologue's normalisation of k (|k_hat|^2 = |k|^2 / |k|^2)
    const float sk = GATE ? inv_norm(n) : 1.f;
    if (GATE) n *= sk * sk;
    const float cn = ok ? (mu / (float(DK) * rt)) * n : 0.f;
    // this token's Mobius matrix [[m00, m01], [m10, m11]], composed over the
    // chunk's tokens by an inclusive scan; G by an inclusive sum
    float m00 = asq, m01 = w, m10 = cn * asq, m11 = fmaf(cn, w, 1.f);
    float g = lg;
    scan_level<kRowShr + 1, 0xf>(m00, m01, m10, m11, g);
    scan_level<kRowShr + 2, 0xf>(m00, m01, m10, m11, g);
    scan_level<kRowShr + 4, 0xf>(m00, m01, m10, m11, g);
    scan_level<kRowShr + 8, 0xf>(m00, m01, m10, m11, g);
    scan_level<kRowBcast15, 0xa>(m00, m01, m10, m11, g);
    const float bt = (m00 * bprev + m01) / (m10 * bprev + m11);  // b after token t
    const float bbefore = dpp<kWaveShr1>(bprev, bt);              // b before token t (lane 0: bprev)
    const float bh = ok ? fmaf(asq, bbefore, w) : 0.f;             // b_hat (padding tokens: no write)
    const float gL = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), L - 1));
    // frame: S_c = gam S~_c.  After the chunk S_{c+1} = 2^G_L S_c + K^T diag(w) Dn.
    // Either the frame absorbs the decay (gam' = gam 2^G_L >= 2^-64, S~ unchanged
    // apart from the write, whose weights are w / gam'), or S~ takes the factor
    // gam 2^G_L (C-input) and gam' = 1.
    const float dL = __builtin_amdgcn_exp2f(gL);
    const float gnext = gam * dL;
    const bool absorb = gnext >= kFrameMin;
    const float wcol = bh * __builtin_amdgcn_exp2f(gL - g);  // w_s
    const int slot = c & 3;
    if (lane < L) {
        const float rw = __builtin_amdgcn_exp2f(g) * gam;  // row weight of R and O: 2^G_t Gamma_c
        sm.sc[slot][0][lane] = rt;
        sm.sc[slot][1][lane] = bh;
        sm.sc[slot][2][lane] = g;
        sm.sc[slot][3][lane] = rw * sk;  // gated: R's rows of K S~ use k_hat = k / |k|
        sm.ws[slot][lane] = (absorb ? wcol * __builtin_amdgcn_rcpf(gnext) : wcol) * sk;
        if (GATE) {
            sm.sc[slot][4][lane] = sk;
            sm.sc[slot][5][lane] = rw;  // times 1/|q_t| by the Gram-P wave
        }
    }
    if (lane == 0) {
        sm.ch[slot][0] = absorb ? 1.f : gnext;  // the update's C-input factor
        sm.ch[slot][1] = gam;                   // the frame at the chunk's start
        sm.ch[slot][2] = absorb ? gnext : 1.f;  // the frame after the chunk
    }
    gam = absorb ? gnext : 1.f;
    bprev = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bt), L - 1));
}

// ---------------------------------------------------------------------------
// direct copies of k, q tiles into LDS ([t][sw(i)]: lane slot P of the tile is
// row P / NCH, 16-byte piece P % NCH of the swizzled row)
// ---------------------------------------------------------------------------
template <int DK>
__device__ __forceinline__ void tile_issue(bf16_t* dst, const bf16_t* src, const IsoArgs& a, int h, int c,
                                           int nchunks) {
    c = min(max(c, 0), nchunks - 1);  // always the same number of copies (the waits count them)
    constexpr int NCH = DK / 8;
    const int lane = threadIdx.x & 63;
    const int last = a.T - 1 - c * L;
    const bf16_t* base = src + tokidx(a, h, c * L) * DK;
    const uint32_t rs = uint32_t(a.H) * DK * 2;
#pragma unroll
    for (int m = 0; m < L * NCH / 64; ++m) {
        const int pc = lane + 64 * m;
        const int row = pc / NCH, slot = pc % NCH;
        const int cg = (slot ^ row) & (NCH - 1);
        const uint32_t off = uint32_t(min(row, last)) * rs + uint32_t(cg) * 16;
        g2lds16(base, off, dst + m * 512);
    }
}
template <int DK>
constexpr int tile_copies() {
    return L * (DK / 8) / 64;
}

// ---------------------------------------------------------------------------
// Gram wave: the chunk's 32 x 32 products on the raw tiles, weighted
// ---------------------------------------------------------------------------
// Row tile ta (16 rows) of a [t][sw(i)] tile as matrix-core operands: lane
// (n, kg8) holds row 16 ta + n, channels 32 kk + kg8 .. + 7.  The same
// registers serve as A (rows of the product) and as B (its columns).
template <int DK>
struct RowTile {
    b8 x[DK / 32];
};
template <int DK>
__device__ __forceinline__ RowTile<DK> row_tile(const bf16_t* A, int ta) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, kg8 = (lane >> 4) * 8;
    RowTile<DK> r;
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) r.x[kk] = *reinterpret_cast<const b8*>(A + sw<DK>(16 * ta + n, 32 * kk + kg8));
    return r;
}
// acc[e] = (A B^T)[g4 + e][n] for 16-row tiles A, B
template <int DK>
__device__ __forceinline__ f4 gram_tile(const RowTile<DK>& A, const RowTile<DK>& B) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) acc = mfma32(A.x[kk], B.x[kk], acc);
    return acc;
}

// the pair weights b_hat_s 2^(G_t - G_s) of tile (ta, tb) for lane (rows
// 16 ta + g4 + e, column 16 tb + n); zero above the diagonal
template <int DK>
__device__ __forceinline__ f4 pair_weights(const IsoSmem<DK>& sm, int slot, int ta, int tb) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = (lane >> 4) * 4;
    const int s = 16 * tb + n;
    const float bs = sm.sc[slot][1][s], gs = sm.sc[slot][2][s];
    const f4 gt = *reinterpret_cast<const f4*>(&sm.sc[slot][2][16 * ta + g4]);
    f4 wv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int t = 16 * ta + g4 + e;
        wv[e] = t >= s ? bs * __builtin_amdgcn_exp2f(gt[e] - gs) : 0.f;
    }
    return wv;
}

// the prologue's key scales of a tile pair (gated): 1/|k_t| of rows 16 ta + g4 + e
// times 1/|k_s| of column 16 tb + n
template <int DK>
__device__ __forceinline__ f4 key_scales(const IsoSmem<DK>& sm, int slot, int ta, int tb) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = (lane >> 4) * 4;
    const f4 st = *reinterpret_cast<const f4*>(&sm.sc[slot][4][16 * ta + g4]);
    const float ss = sm.sc[slot][4][16 * tb + n];
    return f4{st[0] * ss, st[1] * ss, st[2] * ss, st[3] * ss};
}

// M's diagonal blocks (fp32, column-major) and -M_10 (bf16) of the chunk in slot `slot`
template <int DK, bool GATE>
__device__ __forceinline__ void gram_m(IsoSmem<DK>& sm, int kslot, int slot, int md, int mo) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = (lane >> 4) * 4;
    const RowTile<DK> k0 = row_tile<DK>(sm.K[kslot], 0), k1 = row_tile<DK>(sm.K[kslot], 1);
#pragma unroll
    for (int a = 0; a < NT; ++a) {
        const f4 acc = gram_tile<DK>(a ? k1 : k0, a ? k1 : k0);
        f4 wv = pair_weights<DK>(sm, slot, a, a);
        if (GATE) wv *= key_scales<DK>(sm, slot, a, a);
        const f4 rv = *reinterpret_cast<const f4*>(&sm.sc[slot][0][16 * a + g4]);
        f4 mv;
#pragma unroll
        for (int e = 0; e < 4; ++e) mv[e] = fmaf(wv[e], acc[e], g4 + e == n ? rv[e] : 0.f);
        *reinterpret_cast<f4*>(&sm.Md[md][a * 256 + n * 16 + g4]) = mv;
    }
    const f4 acc = gram_tile<DK>(k1, k0);
    f4 wv = pair_weights<DK>(sm, slot, 1, 0);
    if (GATE) wv *= key_scales<DK>(sm, slot, 1, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.Mo[mo][(g4 + e) * 16 + n] = to_bf(-wv[e] * acc[e]);
}

// |x|^2 of row 16 ta + n of a row tile, in every lane of column n
template <int DK>
__device__ __forceinline__ float row_sumsq(const RowTile<DK>& t) {
    float s = 0.f;
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = static_cast<float>(t.x[kk][j]);
            s = fmaf(x, x, s);
        }
    s = halve16(s, s);
    return halve32(s, s);
}

// P = tril(weighted Q K^T) of the chunk, bf16 [t][perm32(s)].  Gated: the
// prologue's 1/|q_t| (from the q tiles, here) and 1/|k_s| go into P's
// weights, and 1/|q_t| into O's row weights.
template <int DK, bool GATE>
__device__ __forceinline__ void gram_p(IsoSmem<DK>& sm, int kslot, int slot, int pslot) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = (lane >> 4) * 4;
    const RowTile<DK> k0 = row_tile<DK>(sm.K[kslot], 0), k1 = row_tile<DK>(sm.K[kslot], 1);
    const RowTile<DK> q0 = row_tile<DK>(sm.Q[kslot], 0), q1 = row_tile<DK>(sm.Q[kslot], 1);
    const f4 a00 = gram_tile<DK>(q0, k0), a10 = gram_tile<DK>(q1, k0), a11 = gram_tile<DK>(q1, k1);
    f4 w00 = pair_weights<DK>(sm, slot, 0, 0), w10 = pair_weights<DK>(sm, slot, 1, 0),
       w11 = pair_weights<DK>(sm, slot, 1, 1);
    if (GATE) {
        const float sq0 = inv_norm(row_sumsq<DK>(q0)), sq1 = inv_norm(row_sumsq<DK>(q1));
        if (lane < 16) {
            sm.qn[n] = sq0;
            sm.qn[16 + n] = sq1;
            sm.sc[slot][5][n] *= sq0;
            sm.sc[slot][5][16 + n] *= sq1;
        }
        wave_lds_sync();
        const f4 qa0 = *reinterpret_cast<const f4*>(&sm.qn[g4]), qa1 = *reinterpret_cast<const f4*>(&sm.qn[16 + g4]);
        const float ks0 = sm.sc[slot][4][n], ks1 = sm.sc[slot][4][16 + n];
        w00 *= qa0 * ks0;
        w10 *= qa1 * ks0;
        w11 *= qa1 * ks1;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        sm.P[pslot][(g4 + e) * PT + perm32(n)] = to_bf(w00[e] * a00[e]);
        sm.P[pslot][(16 + g4 + e) * PT + perm32(n)] = to_bf(w10[e] * a10[e]);
        sm.P[pslot][(16 + g4 + e) * PT + perm32(16 + n)] = to_bf(w11[e] * a11[e]);
    }
}
// Not gated, in two parts on two waves: tiles (0,0) and (1,0) of P, then
// tile (1,1), each reading only the row tiles it needs.
template <int DK>
__device__ __forceinline__ void gram_p_part(IsoSmem<DK>& sm, int kslot, int slot, int pslot, int part) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = (lane >> 4) * 4;
    if (part == 0) {
        const RowTile<DK> k0 = row_tile<DK>(sm.K[kslot], 0);
        const RowTile<DK> q0 = row_tile<DK>(sm.Q[kslot], 0), q1 = row_tile<DK>(sm.Q[kslot], 1);
        const f4 a00 = gram_tile<DK>(q0, k0), a10 = gram_tile<DK>(q1, k0);
        const f4 w00 = pair_weights<DK>(sm, slot, 0, 0), w10 = pair_weights<DK>(sm, slot, 1, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sm.P[pslot][(g4 + e) * PT + perm32(n)] = to_bf(w00[e] * a00[e]);
            sm.P[pslot][(16 + g4 + e) * PT + perm32(n)] = to_bf(w10[e] * a10[e]);
        }
    } else {
        const RowTile<DK> k1 = row_tile<DK>(sm.K[kslot], 1), q1 = row_tile<DK>(sm.Q[kslot], 1);
        const f4 a11 = gram_tile<DK>(q1, k1);
        const f4 w11 = pair_weights<DK>(sm, slot, 1, 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.P[pslot][(16 + g4 + e) * PT + perm32(16 + n)] = to_bf(w11[e] * a11[e]);
    }
}


// ---------------------------------------------------------------------------
// state: one wave = 16 value columns, S~ (d_k x 16 fp32) in registers
// ---------------------------------------------------------------------------
// Register row p of S~ (p = 16 it + g4 + e in the accumulator layout) holds
// key channel chan_of(p): within each block of 32, rows 4g..4g+3 hold
// channels 8g..8g+3 and rows 16+4g..16+4g+3 channels 8g+4..8g+7.  The bf16
// operand built from rows {32kk + 4g + e, 32kk + 16 + 4g + e} then covers the
// 8 consecutive channels 32kk + 8g.. that lane group g reads from a k or q
// tile in natural order, and k^T is stored in the same row order.
__device__ __forceinline__ int chan_of(int p) {
    const int q = p & 31;
    return (p & ~31) + (q < 16 ? 8 * (q >> 2) + (q & 3) : 8 * ((q - 16) >> 2) + 4 + (q & 3));
}
// 16-byte unit of k^T: the low two bits XOR bits 5..6.  The transpose's
// lanes (cg) write units 32 (cg >> 2) + 4 (cg & 3) + j, which would share
// four bank groups; the state waves read 16 consecutive units, for which the
// XOR is one constant.
__device__ __forceinline__ int kt_unit(int u) { return u ^ ((u >> 5) & 3); }
__device__ __forceinline__ int pos_of(int ch) {
    const int j = ch & 7, g = (ch >> 3) & 3;
    return (ch & ~31) + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4);
}
// k^T of a chunk for the update's A operand, rows in the state's order:
// lane (q = lane >> 4, channel group cg = lane & 15) transposes the 8 x 8
// block of tokens {4q..4q+3, 16+4q..+3} and channels 8 cg .. 8 cg + 7
// (DK = 64: lanes with cg < 8)
template <int DK>
__device__ __forceinline__ void transpose_k(bf16_t* KT, const bf16_t* K) {
    const int lane = threadIdx.x & 63;
    const int qg = lane >> 4, cg = lane & 15;
    if (cg >= DK / 8) return;
    u4 rw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int t = (j < 4 ? 4 * qg + j : 16 + 4 * qg + j - 4);
        rw[j] = *reinterpret_cast<const u4*>(K + sw<DK>(t, 8 * cg));
    }
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
        const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
        u4 outv;
#pragma unroll
        for (int m = 0; m < 4; ++m) outv[m] = __builtin_amdgcn_perm(rw[2 * m + 1][cc >> 1], rw[2 * m][cc >> 1], sel);
        *reinterpret_cast<u4*>(KT + kt_unit(qg * DK + pos_of(8 * cg + cc)) * 8) = outv;
    }
}

// A state wave holds NCW tiles of 16 value columns: S~ (d_k x 16 NCW fp32)
// in registers, tile j in S[j]
template <int DK, int NCW>
struct IsoState {
    f4 S[NCW][DK / 16];   // rows 16 it + g4 + e, column 16 j + n
    b8 Sb[NCW][DK / 32];  // bf16 operands of S~
};
template <int DK, int NCW>
__device__ __forceinline__ void iso_pack(IsoState<DK, NCW>& st) {
#pragma unroll
    for (int j = 0; j < NCW; ++j)
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) st.Sb[j][kk] = pack8(st.S[j][2 * kk], st.S[j][2 * kk + 1]);
}

// v tile (32 tokens x 16 NCW columns) of chunk c (clamped into the sequence)
// into state wave sw_'s part of RV[slot]: NCW copies of 64 pieces
template <int DK, int NCW>
__device__ __forceinline__ void v_issue(IsoSmem<DK>& sm, const IsoArgs& a, int h, int col0, int sw_, int c,
                                        int slot, int nchunks) {
    c = min(max(c, 0), nchunks - 1);
    const int lane = threadIdx.x & 63;
    const int last = a.T - 1 - c * L;
    const bf16_t* base = a.v + tokidx(a, h, c * L) * a.DV + col0;
    const uint32_t rs = uint32_t(a.H) * uint32_t(a.DV) * 2;
#pragma unroll
    for (int m = 0; m < NCW; ++m) {
        const int pc = lane + 64 * m, row = pc / (2 * NCW), piece = pc % (2 * NCW);
        const uint32_t off = uint32_t(min(row, last)) * rs + uint32_t(piece) * 16;
        g2lds16(base, off, &sm.RV[slot][(sw_ * NCW + m) * 512]);
    }
}

// The k and q rows of a state chunk as matrix-core operands (lane (n, kg8):
// row 16 at + n, channels 32 kk + kg8 .. + 7).  A state wave loads the next
// chunk's during the S update of the current one, so the reads overlap
// those products instead of opening the next chunk.
template <int DK>
struct StateOps {
    b8 ak[NT][DK / 32], aq[NT][DK / 32];
};
template <int DK>
__device__ __forceinline__ void iso_ops_load(StateOps<DK>& op, const IsoSmem<DK>& sm, int c) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, kg8 = (lane >> 4) * 8;
    const int kslot = c % KR;
#pragma unroll
    for (int at = 0; at < NT; ++at)
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            op.ak[at][kk] = *reinterpret_cast<const b8*>(sm.K[kslot] + sw<DK>(16 * at + n, 32 * kk + kg8));
            op.aq[at][kk] = *reinterpret_cast<const b8*>(sm.Q[kslot] + sw<DK>(16 * at + n, 32 * kk + kg8));
        }
}

template <int NCW>
struct SegCarry {
    f4 O[NCW][NT];  // (Q S)^T of the chunk, scaled: value column x token
    b8 Db[NCW];     // Dn (bf16, A operand) for P Dn
    b8 Dw[NCW];     // diag(w) Dn for the update
};

template <int DK, int NCW, bool GATE>
__device__ __forceinline__ void iso_seg1(IsoState<DK, NCW>& st, SegCarry<NCW>& cy, IsoSmem<DK>& sm, int c,
                                         int sw_, const StateOps<DK>& op) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = (lane >> 4) * 4;
    constexpr int KS = DK / 32;
    constexpr int VP = 16 * NCW;  // v row pitch
    const int slot = c & 3, vslot = c % 3, mb = c & 1, m3 = c % 3;
    const bf16_t* rv = &sm.RV[vslot][sw_ * NCW * 512];
    // read phase (the k and q operands came with op)
    const auto& ak = op.ak;
    const auto& aq = op.aq;
    uint32_t vr[NCW][NT][4];
    f4 rw[NT];
#pragma unroll
    for (int at = 0; at < NT; ++at) {
#pragma unroll
        for (int j = 0; j < NCW; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) vr[j][at][e] = rv[(16 * at + g4 + e) * VP + 16 * j + n];
        rw[at] = *reinterpret_cast<const f4*>(&sm.sc[slot][3][16 * at + g4]);
    }
    // O's row weights (gated: with 1/|q_t|; otherwise R's)
    const float rq0 = sm.sc[slot][GATE ? 5 : 3][n], rq1 = sm.sc[slot][GATE ? 5 : 3][16 + n];
    const f4 wc0 = *reinterpret_cast<const f4*>(&sm.ws[slot][g4]);
    const f4 wc1 = *reinterpret_cast<const f4*>(&sm.ws[slot][16 + g4]);
    const s4 t0 = *reinterpret_cast<const s4*>(&sm.Td[mb][n * 16 + g4]);
    const s4 t1 = *reinterpret_cast<const s4*>(&sm.Td[mb][256 + n * 16 + g4]);
    const s4 mo = *reinterpret_cast<const s4*>(&sm.Mo[m3][n * 16 + g4]);
#pragma unroll
    for (int j = 0; j < NCW; ++j) {
        f4 R[NT];
#pragma unroll
        for (int at = 0; at < NT; ++at) {
            f4 ks = {0.f, 0.f, 0.f, 0.f}, o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                ks = mfma32(ak[at][kk], st.Sb[j][kk], ks);  // K S~: token x value column
                o = mfma32(st.Sb[j][kk], aq[at][kk], o);    // (Q S~)^T: value column x token
            }
            // R = V - diag(2^G Gamma) K S~,  O = diag(2^G Gamma) Q S~
#pragma unroll
            for (int e = 0; e < 4; ++e) R[at][e] = fmaf(-rw[at][e], ks[e], bf1(bf16_t(vr[j][at][e])));
            const float rq = at ? rq1 : rq0;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] *= rq;
            cy.O[j][at] = o;
        }
        // Dn = M^-1 R by block substitution
        const f4 zero = {0.f, 0.f, 0.f, 0.f};
        const f4 d0 = mfma16(t0, pack4(R[0]), zero);
        const f4 r1 = mfma16(mo, pack4(d0), R[1]);
        const f4 d1 = mfma16(t1, pack4(r1), zero);
        cy.Db[j] = pack8(d0, d1);
        f4 e0, e1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            e0[e] = d0[e] * wc0[e];
            e1[e] = d1[e] * wc1[e];
        }
        cy.Dw[j] = pack8(e0, e1);
    }
}

template <int DK, int NCW>
__device__ __forceinline__ void iso_seg2(IsoState<DK, NCW>& st, const SegCarry<NCW>& cy, IsoSmem<DK>& sm,
                                         const IsoArgs& a, int h, int col0, int c, int nchunks,
                                         StateOps<DK>& op) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = (lane >> 4) * 4, kg8 = (lane >> 4) * 8;
    const int slot = c & 3;
    const bool full = (c + 1) * L <= a.T;
    b8 ap[NT], akt[DK / 16];
#pragma unroll
    for (int at = 0; at < NT; ++at) ap[at] = *reinterpret_cast<const b8*>(&sm.P[c % 3][(16 * at + n) * PT + kg8]);
#pragma unroll
    for (int it = 0; it < DK / 16; ++it)
        akt[it] = *reinterpret_cast<const b8*>(&sm.KT[c & 1][kt_unit((lane >> 4) * DK + 16 * it + n) * 8]);
    const float cin = sm.ch[slot][0];
    // outputs, transposed: lane (n, g4) holds value columns 16 j + g4 .. + 3 of token 16 at + n
    bf16_t* orow = a.o + tokidx(a, h, c * L + n) * a.DV + col0 + g4;
    const size_t ostep = size_t(16) * a.H * a.DV;
#pragma unroll
    for (int at = 0; at < NT; ++at) {
#pragma unroll
        for (int j = 0; j < NCW; ++j) {
            const f4 o = mfma32(cy.Db[j], ap[at], cy.O[j][at]);  // + (P Dn)^T
            if (full || c * L + 16 * at + n < a.T)
                *reinterpret_cast<u2*>(orow + 16 * j) = u2{pack2(o[0], o[1]), pack2(o[2], o[3])};
        }
        orow += ostep;
    }
    // the next chunk's k and q operands (its tiles landed iterations ago;
    // their ring slot is not reused before the next chunk is done)
    if (c + 1 < nchunks) iso_ops_load<DK>(op, sm, c + 1);
    // S~ <- cin S~ + K^T diag(w') Dn  (cin = 1 unless the frame is renormalised)
    if (cin != 1.f) {
#pragma unroll
        for (int j = 0; j < NCW; ++j)
#pragma unroll
            for (int it = 0; it < DK / 16; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e) st.S[j][it][e] *= cin;
    }
#pragma unroll
    for (int it = 0; it < DK / 16; ++it)
#pragma unroll
        for (int j = 0; j < NCW; ++j) st.S[j][it] = mfma32(akt[it], cy.Dw[j], st.S[j][it]);
    iso_pack<DK, NCW>(st);
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int DK, int NSW, bool GATE>
__global__ void __launch_bounds__(NTHREADS) kdn_iso_kernel(IsoArgs a) {
    constexpr int NCW = 1;                // 16-column tiles per state wave
    constexpr int DVTN = 16 * NSW * NCW;  // value columns of this workgroup
    __shared__ IsoSmem<DK> sm;
    const int ntile = a.DV / DVTN;
    const int bid = blockIdx.x;
    // work items dealt to the eight XCDs in turn, batch-fastest; the column
    // tiles of one (batch, head) share an XCD
    const int item = (bid / (8 * ntile)) * 8 + (bid % 8);
    const int tile = (bid / 8) % ntile;
    if (item >= a.units) return;
    const int nbatch = a.units / a.H;
    int h = item / nbatch;
    size_t b = size_t(item % nbatch);
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int lane = threadIdx.x & 63;
    if (a.cu) {
        h = item % a.H;
        const int rank = item / a.H;
        b = size_t(a.ord ? min(max(a.ord[rank], 0), nbatch - 1) : rank);
        const int total = a.T;
        const int s0 = min(max(a.cu[b], 0), total);
        const int s1 = min(max(a.cu[b + 1], s0), total);
        a.tok0 = size_t(s0);
        a.T = s1 - s0;
    } else {
        a.tok0 = b * size_t(a.T);
    }
    const int unit = int(b) * a.H + h;
    if (a.T == 0) {
        const size_t sb = size_t(unit) * DK * a.DV;
        for (int e = threadIdx.x; e < DK * DVTN; e += NTHREADS) {
            const size_t x = sb + size_t(e / DVTN) * a.DV + tile * DVTN + e % DVTN;
            a.S_T[x] = a.S0 ? a.S0[x] : 0.f;
        }
        if (tile == 0 && threadIdx.x == 0) a.p_T[unit] = a.p0 ? a.p0[unit] : a.c0[h];
        return;
    }
    const int nchunks = (a.T + L - 1) / L;
    // iteration i: scan of chunk i, Gram products of chunk i - 1, inverses and
    // k^T of chunk i - 2, state update of chunk i - 3; one barrier each
    const int nit = nchunks + 3;
    constexpr int NK = 2 * tile_copies<DK>();  // copies per chunk (k and q)

    // the zero upper block of P's first row tile and of each inverse, once
    for (int e = threadIdx.x; e < 3 * 16 * 16; e += NTHREADS) {
        const int s3 = e >> 8, t = (e >> 4) & 15, s = 16 + (e & 15);
        sm.P[s3][t * PT + perm32(s)] = 0;
    }
    for (int e = threadIdx.x; e < 2 * 2 * 64; e += NTHREADS) {
        const int bb = e >> 7, a2 = (e >> 6) & 1, tt = (e >> 3) & 7, ss = 8 + (e & 7);
        sm.Td[bb][a2 * 256 + tt * 16 + ss] = 0;
    }
    if (wave == 3) {
        tile_issue<DK>(sm.K[0], a.k, a, h, 0, nchunks);
        tile_issue<DK>(sm.Q[0], a.q, a, h, 0, nchunks);
        tile_issue<DK>(sm.K[1], a.k, a, h, 1, nchunks);
        tile_issue<DK>(sm.Q[1], a.q, a, h, 1, nchunks);
        vm_wait<NK>();  // chunk 0 has landed
        if (!GATE) {
            const float nrm = tile_norm<DK>(sm.K[0]);
            if (lane < L) sm.kn[0][lane] = nrm;
        }
    }
    bar();

    if (wave == 0) {
        // ---------------- scan of chunk i ----------------
        float bprev = a.p0 ? a.p0[unit] : a.c0[h];
        float gam = 1.f;  // the state's frame
        ScanRegs X;
        scan_load(X, a, h, 0, nchunks);
        for (int i = 0; i < nit; ++i) {
            if (i < nchunks) {
                // gated: the q norms load the copy wave, so the scan takes the k norms itself
                const float nrm = GATE ? tile_norm<DK>(sm.K[i % KR]) : sm.kn[i & 1][lane & 31];
                scan_run<DK, GATE>(X, sm, i, nrm, a.mu, bprev, gam, min(L, a.T - i * L));
            }
            scan_load(X, a, h, i + 1, nchunks);  // used at the next iteration
            bar();
        }
        if (lane == 0 && tile == 0) a.p_T[unit] = bprev;
    } else if (wave == 1) {
        // ---------------- M of chunk i - 1; k^T of chunk i - 2 ----------------
        for (int i = 0; i < nit; ++i) {
            const int c = i - 1;
            if (c >= 0 && c < nchunks) gram_m<DK, GATE>(sm, c % KR, c & 3, c & 1, c % 3);
            if (!GATE && c >= 0 && c < nchunks) gram_p_part<DK>(sm, c % KR, c & 3, c % 3, 1);
            if (c >= 1 && c <= nchunks) transpose_k<DK>(sm.KT[(c - 1) & 1], sm.K[(c - 1) % KR]);
            bar();
        }
    } else if (wave == 2) {
        // ---------------- inverses of chunk i - 2; (not gated) P of chunk i - 1 ----------------
        for (int i = 0; i < nit; ++i) {
            const int c = i - 2;
            if (c >= 0 && c < nchunks) block_inverse(sm.Md[c & 1], sm.Wi, sm.Td[c & 1], lane);
            if (!GATE && c + 1 >= 0 && c + 1 < nchunks) gram_p_part<DK>(sm, (c + 1) % KR, (c + 1) & 3, (c + 1) % 3, 0);
            bar();
        }
    } else if (wave == 3) {
        // ---------------- tile copies; |k|^2 of chunk i + 1; P of chunk i - 1 ----------------
        for (int i = 0; i < nit; ++i) {
            // chunk i + 2 into slot (i + 2) % KR: its previous occupant, chunk
            // i + 2 - KR, was last read at iteration i - 1
            tile_issue<DK>(sm.K[(i + 2) % KR], a.k, a, h, i + 2, nchunks);
            tile_issue<DK>(sm.Q[(i + 2) % KR], a.q, a, h, i + 2, nchunks);
            vm_wait<NK>();  // chunk i + 1 (copied at iteration i - 1) has landed; chunk i + 2 may not have
            if (!GATE && i + 1 < nchunks) {
                // the row norms the scan takes at iteration i + 1 (its slot was
                // last read at iteration i - 1)
                const float nrm = tile_norm<DK>(sm.K[(i + 1) % KR]);
                if (lane < L) sm.kn[(i + 1) & 1][lane] = nrm;
            }
            const int c = i - 1;
            if (GATE && c >= 0 && c < nchunks) gram_p<DK, GATE>(sm, c % KR, c & 3, c % 3);
            bar();
        }
        vm_wait<0>();
    } else if (wave >= 4 && wave < 4 + NSW) {
        // ---------------- state: chunk i - 3 ----------------
        const int sw_ = wave - 4;
        const int col0 = tile * DVTN + 16 * NCW * sw_;  // first column within the head
        const int n = lane & 15, g4 = (lane >> 4) * 4;
        IsoState<DK, NCW> st;
        SegCarry<NCW> cy;
        StateOps<DK> op;  // k and q operands of the next state chunk
        const size_t sbase = size_t(unit) * DK * a.DV;
#pragma unroll
        for (int j = 0; j < NCW; ++j)
#pragma unroll
            for (int it = 0; it < DK / 16; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    st.S[j][it][e] =
                        a.S0 ? a.S0[sbase + size_t(chan_of(16 * it + g4 + e)) * a.DV + col0 + 16 * j + n] : 0.f;
#pragma unroll
        for (int j = 0; j < NCW; ++j)
#pragma unroll
            for (int it = 0; it < DK / 16; ++it) settle(st.S[j][it]);
        iso_pack<DK, NCW>(st);
        for (int i = 0; i < nit; ++i) {
            const int c = i - 3;
            // v of chunk i - 1 into slot (i - 1) mod 3 = (i + 2) % 3
            v_issue<DK, NCW>(sm, a, h, col0, sw_, i - 1, (i + 2) % 3, nchunks);
            if (c >= 0) {
                // the v of chunk c (copied at iteration i - 2) has landed: the
                // memory counter drains in order, and after that copy come the
                // v copies of iterations i - 1 and i (NCW each) and the NT NCW
                // output stores of iterations i - 2 and i - 1 where those
                // updated a chunk
                constexpr int NV = NCW, NS = NT * NCW;
                if (i >= 5) vm_wait<2 * NS + 2 * NV>();
                else if (i == 4) vm_wait<NS + 2 * NV>();
                else vm_wait<2 * NV>();
                if (c == 0) iso_ops_load<DK>(op, sm, 0);
                iso_seg1<DK, NCW, GATE>(st, cy, sm, c, sw_, op);
                iso_seg2<DK, NCW>(st, cy, sm, a, h, col0, c, nchunks, op);
            }
            bar();
        }
        // S = Gamma S~ with the frame after the last chunk
        const float gam = sm.ch[(nchunks - 1) & 3][2];
        vm_wait<0>();
#pragma unroll
        for (int j = 0; j < NCW; ++j)
#pragma unroll
            for (int it = 0; it < DK / 16; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a.S_T[sbase + size_t(chan_of(16 * it + g4 + e)) * a.DV + col0 + 16 * j + n] = st.S[j][it][e] * gam;
    } else {
        for (int i = 0; i < nit; ++i) bar();
    }
}

template <int DK, int NSW, bool GATE>
hipError_t launch_iso_t(const FwdArgs& f, hipStream_t stream) {
    const int units = f.B * f.H;
    if (units == 0) return hipSuccess;
    IsoArgs a;
    a.q = static_cast<const bf16_t*>(f.q);
    a.k = static_cast<const bf16_t*>(f.k);
    a.v = static_cast<const bf16_t*>(f.v);
    a.alpha = static_cast<const bf16_t*>(f.alpha);
    a.omega = static_cast<const bf16_t*>(f.omega);
    a.r = static_cast<const bf16_t*>(f.r);
    a.c0 = f.c0;
    a.mu = f.mu;
    a.T = f.T;
    a.H = f.H;
    a.DV = f.dv;
    a.units = units;
    a.S0 = f.S0;
    a.p0 = f.p0;
    a.o = static_cast<bf16_t*>(f.o);
    a.S_T = f.S_T;
    a.p_T = f.p_T;
    a.cu = f.cu_seqlens;
    a.ord = f.seq_order;
    a.tok0 = 0;
    const int ntile = f.dv / (16 * NSW);
    const int groups = (units + 7) / 8;
    const unsigned grid = unsigned(groups) * 8u * unsigned(ntile);
    hipLaunchKernelGGL((kdn_iso_kernel<DK, NSW, GATE>), dim3(grid), dim3(NTHREADS), 0, stream, a);
    return hipGetLastError();
}

template <int DK, bool GATE>
hipError_t launch_iso_dk(const FwdArgs& a, bool narrow, hipStream_t stream) {
    return narrow ? launch_iso_t<DK, 2, GATE>(a, stream) : launch_iso_t<DK, 4, GATE>(a, stream);
}

}  // namespace

hipError_t launch_iso(const FwdArgs& a, bool narrow, hipStream_t stream) {
    if (a.variant != 1) return hipErrorNotSupported;
    if (a.dk == 128) return a.gates ? launch_iso_dk<128, true>(a, narrow, stream) : launch_iso_dk<128, false>(a, narrow, stream);
    if (a.dk == 64) return a.gates ? launch_iso_dk<64, true>(a, narrow, stream) : launch_iso_dk<64, false>(a, narrow, stream);
    return hipErrorNotSupported;
}

}  // namespace kdn
