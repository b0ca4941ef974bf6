// kdn_chunked.hip -- chunkwise forward of the KDN recurrence on gfx950: a
// pipelined, wave-specialised kernel with the token-to-token coupling on
// matrix cores (MFMA) and the fp32 memory carried in registers.
//
// Method ("Kalman Delta Networks: Uncertainty-aware Associative Memory",
// summary page, method steps 2-5 and the isotropic closing sentence).  Per
// (batch, head) and token t, with fp32 state:
//   p_hat = alpha^2 * p + omega;  kappa = p_hat * k / (r + sum_i p_hat_i k_i^2)
//   S = diag(alpha) S + kappa (v - (diag(alpha) S)^T k)^T;  o = S^T q
//   p = p_hat / (1 + (mu / r) k^2 p_hat)
//
// Chunk form (our derivation from those steps).  The sequence is cut into
// chunks of L = 32 tokens.  Inside a chunk the decay from token s to a later
// token t is prod_{s<u<=t} alpha_u (per key channel).  It is factored as
// rho_t / rho_s with rho referenced to the chunk's midpoint (between tokens
// 15 and 16): with g_t = prod_{u<=t} alpha_u from the chunk start,
//   rho_t = g_t / g_15 (t <= 15),   rho_t = prod_{16<=u<=t} alpha_u (t >= 16),
// so rho_t >= 1 in the first half and <= 1 in the second, and no factor spans
// more than one 16-token half.  With kappa'_t = p_hat_t * k_t the gain
// numerator, d_t = r_t + sum_i p_hat_t,i k_t,i^2 its denominator,
//   Kt_t = k_t rho_t,  Qt_t = q_t rho_t,  Kh_t = kappa'_t / rho_t,
//   Sg = diag(g_15) S_c,  Dn_t = (v_t - (diag(alpha_t) S_{t-1})^T k_t) / d_t,
// the chunk's writes satisfy
//   M Dn = V - Kt Sg,        M = diag(r) + tril(Kt Kh^T)  (diagonal included:
//                                                        M_tt = d_t)
//   O    = Qt Sg + tril(Qt Kh^T) Dn
//   S_{c+1} = diag(gb_31) (Sg + Kh^T Dn),   gb_31 = prod_{16<=u<=31} alpha_u
// which is the token recurrence rewritten exactly.  M is lower triangular;
// its two 16 x 16 diagonal blocks are inverted in fp32 and the solve is a
// two-step block substitution on MFMA.  Operands are bf16 with fp32
// accumulation; S, p and every scalar recurrence stay fp32.
//
// Range.  The largest factor is 1 / (the decay over one half-chunk), on
// either side, and every product used (t >= s) is at most |k| |kappa'|.  A
// chunk whose half-chunk decays g_15 or gb_31 fall below 2^-96 on some
// channel is outside this form's range: the chain flags it, every role stops
// after the chunk before it, and the workgroup finishes its sequence with the
// token recurrence (kdn_recurrent_core.h) from that chunk on, from the state
// the chunked form carried to it.  Results are then exact for every
// 0 < alpha <= 1, and the chunked form covers decays down to a geometric mean
// of about 2^-6 per token (alpha ~ 0.015).

// The uncertainty recurrence is a Mobius map of p (summary page, step 5):
// p_t = (a p + w) / (u a p + 1 + u w) with a = alpha^2, w = omega, u = mu k^2 / r.
//  - Diagonal variant: 128 independent channels per head fill a wave's lanes,
//    so each lane runs its channel's map sequentially (one fma, one fma, one
//    reciprocal, one multiply per token); this is the cheapest form in issued
//    instructions, several times cheaper than a cross-lane scan over tokens.
//  - Isotropic variant: one scalar per head, so the maps of a chunk's 32
//    tokens (one per lane) are composed as 2 x 2 matrix products by an
//    inclusive cross-lane scan (5 shuffle levels, renormalised each level).
//  - Isotropic variant with per-channel decay (the general form of that
//    sentence: diag(alpha) on the memory, a = mean_i alpha_i^2 on the
//    uncertainty scalar): the isotropic scan with a, plus a decay chain
//    (wave 1) for the per-channel cumulative decays.
//
// Workgroup = one (batch, head) pair and 64 value columns, 8 waves in roles:
//   waves 0,1      "chain":     uncertainty recurrence of chunk c+2 -> scaled
//                               gains Kh (stored as Kh^T, the state's operand)
//                               and decays g (LDS)
//   waves 2,3,6,7  "formation": MFMA operands Kt, Qt, Kh (isotropic: also
//                               Kh^T) of chunk c+1, then M, tril(Qt Kh^T) and
//                               the diagonal-block inverses of M
//   waves 4,5      "state":     memory pass of chunk c: 32 value columns each,
//                               S (d_k x 32 fp32) in registers
// Two workgroup barriers per iteration; every LDS buffer that crosses an
// iteration is double buffered, and global inputs are prefetched into
// registers one iteration ahead.  Roles run on all four SIMDs so the chain's
// VALU work overlaps the MFMA work of the other roles.
#include "kdn_gates.h"
#include "kdn_device.h"
#include "kdn_internal.h"
#include "kdn_recurrent_core.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstddef>
#include <cstdint>
#include <utility>

namespace kdn {
namespace {

using namespace dev;

constexpr int L = 32;            // tokens per chunk
constexpr int NT = L / 16;       // 16-token tiles per chunk
constexpr int DVT = 64;          // value columns per workgroup (two state waves x two 16-column tiles)
// A narrow workgroup (NCT = 1: one 16-column tile per state wave, 32 value
// columns) doubles the workgroups of a head for batches too small to fill the
// CUs; chain and formation work is per head, so it is repeated per tile.
template <int NCT>
__host__ __device__ constexpr int dvt_of() { return 32 * NCT; }
constexpr int NTHREADS = 512;    // 8 waves
constexpr int PT = L + 8;        // pitch (elements) of [rows][L] bf16 tiles
constexpr int CHAIN_SPLIT = 16;  // chain tokens run before the mid-iteration barrier
static_assert(L == 32 && NT == 2, "the kernel is written for 32-token chunks");

template <int DK>
struct Smem {
    // The chain's tiles come first: every per-token offset into them then
    // fits the 16-bit immediate of the LDS instructions (a larger one makes
    // the compiler keep one address register per token).
    alignas(16) bf16_t RK[2][L * DK];    // raw k, alpha, omega tiles of the chain's next chunk,
    alignas(16) bf16_t RA[2][L * DK];    // [t][i] as in global memory (direct global -> LDS loads)
    alignas(16) bf16_t RW[2][L * DK];
    alignas(16) bf16_t GQ[2][L * DK];    // g_t,i (diagonal variant)  [t / 8][i][t % 8]
    alignas(16) float cr[2][64];         // mu / r_t of the chain's chunks (lane t)
    alignas(16) float ks[2][L];          // gated: 1 / |k_t| of the chain's chunks (the prologue's normalisation)
    alignas(16) float qs[2][L];          // gated: 1 / |q_t| (formed with the chunk, applied to its outputs)
    alignas(16) float gL[3][DK];         // gb_31, the second half's decay, fp32 (ring of three chunks)
    alignas(16) float g15[3][DK];        // g_15, the first half's decay, fp32 (ring of three chunks)
    alignas(16) float fL[3][DK];         // gb_31 of chunk c times g_15 of chunk c + 1 (slot c % 3)
    int fsub[3][2];                      // fL of slot c % 3 is below 2^-124 on some channel (per chain wave)
    alignas(16) bf16_t Kh[L * DK];       // kappa'_t / g_t    [t][perm32(i)], swizzled (read in the same iteration)
    alignas(16) bf16_t Kn[2][L * DK];    // -k_t g_t           [t][perm32(i)], swizzled
    alignas(16) bf16_t Qt[2][L * DK];    //  q_t g_t
    alignas(16) bf16_t KhQ[3][L * DK];   // (kappa'_t / g_t)^T  [P / 8][i][P % 8] with P = perm32(t) (ring of three)
    alignas(16) bf16_t QK[2][L * PT];    // tril(Qt Kh^T)      [t][perm32(s)]
    alignas(16) bf16_t Td[2][NT * 256];  // inverses of M's diagonal blocks [a][t][s]
    alignas(16) bf16_t Mo[2][256];       // -M's block (1,0)   [t][s]
    alignas(16) bf16_t RV[3][2][L * 32]; // v tiles of the two state waves, [t][32 columns], ring of 3
    alignas(16) float rr[3][L];          // r_t (ring of three chunks: written a chunk ahead)
    alignas(16) float bh[2][L];          // b_hat_t (isotropic)
    alignas(16) float gs[2][L];          // g_t (isotropic, scalar)
    alignas(16) float Md[NT * 256];      // M's diagonal blocks, column-major [a][s][t] (fp32)
    alignas(16) float Wi[NT][2][64];     // inverses of their 8x8 diagonal sub-blocks, column-major
    int bad;                             // first chunk outside the chunked form's range (INT_MAX: none)
};

// Smallest half-chunk decay the chunked form accepts (see the range note at
// the top): factors up to 2^96 leave 2^31 of headroom below the bf16 / fp32
// maximum for |k|, |q| and |kappa'|.
constexpr float kRangeMin = 0x1p-96f;

// After the chunked roles stop, the start of the LDS block (the chain's raw
// tiles, idle by then) holds the hand-off to the token recurrence: the memory
// of the workgroup's columns, the uncertainty, and the recurrence's per-wave
// staging slices.
template <int DK>
struct Handoff {
    float S[DK][64];
    float p[DK];
    float4 chan[2][DK];
};

struct Args {
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
    const int* cu;   // packed sequences: sequence n owns tokens [cu[n], cu[n + 1]); NULL: B x T
    const int* ord;  // packed sequences: scheduling order of the sequences, or NULL
    size_t tok0;    // set per workgroup: the first token of its sequence in the token grid
    // segment mode (seg > 0; diagonal, ungated): every sequence is cut into
    // nseg segments of seg tokens, run concurrently.  Column tiles below
    // vtiles hold v columns; the d_k tiles from vtiles on hold the identity
    // columns (start I, v = 0) that carry the segment's state transition.
    // Segment g starts from S = 0 (g > 0) or S0, and from the uncertainty its
    // predecessors' Mobius products (mob) carry p0 to.
    int seg = 0, nseg = 1, vtiles = 0;
    const float* mob = nullptr;  // [B*H][nseg][DK][4] Mobius products of the segments
    bf16_t* ophi = nullptr;      // o of the identity columns, [tokens][H][DK]
    float* sseg = nullptr;       // segment end states [B*H][nseg][DK][DV + DK]
    // checkpoint mode (the chunked backward's forward sweep; diagonal, 64-column
    // tiles): the memory in the midpoint frame, diag(g_15) S, in bf16 at every
    // chunk start ([unit][tile][chunk][DK / 4][64][4] at cks), and p at every
    // chunk start ([unit][chunk][DK] at ckp); ck_flag[unit] = 1 where a chunk
    // leaves the chunked form's range (its checkpoints stop there), else 0.
    // No o, S_T or p_T.
    bf16_t* cks = nullptr;
    float* ckp = nullptr;
    int* ck_flag = nullptr;
};

// position of token t of the workgroup's sequence (of head h) in the token
// grid [tokens, H] (the sequence's tokens are consecutive rows of it)
__device__ __forceinline__ size_t tokidx(const Args& a, size_t, int h, int t) {
    return (a.tok0 + size_t(t)) * size_t(a.H) + size_t(h);
}

// ---------------------------------------------------------------------------
// chain role, diagonal variant: lane = key channel
// ---------------------------------------------------------------------------
// Issue rows 16 HALF .. 16 HALF + 15 of the raw k, alpha, omega tiles of
// chunk c (the chain's input) into LDS buffer c & 1, split over NW issuing
// waves (w = 0 .. NW - 1).  Rows 0..15 of a buffer are free once the chain's
// first segment has read them, so they are fetched one segment earlier than
// rows 16..31, by other waves.  Rows past the end of the sequence repeat the
// last token (masked where used).
template <int DK, int HALF, int NW>
__device__ __forceinline__ void chain_diag_issue(Smem<DK>& sm, const Args& a, size_t b, int h, int c,
                                                 int nchunks, int w) {
    if (c < 0 || c >= nchunks) return;
    constexpr int PR = DK / 8;          // 16-byte pieces per row
    constexpr int NB = L * PR / 64;     // 64-piece blocks per tile (four rows each at d_k = 128)
    constexpr int B0 = HALF * NB / 2, B1 = B0 + NB / 2;
    const int lane = threadIdx.x & 63;
    const int buf = c & 1;
    const int last = a.T - 1 - c * L;                  // last real row of the chunk (>= 0)
    const size_t row0 = tokidx(a, b, h, c * L) * DK;  // the chunk's first row
    const uint32_t rs = uint32_t(a.H) * DK * 2;        // bytes from one token's row to the next
#pragma unroll
    for (int blk = B0 + w; blk < B1; blk += NW) {
        const int pc = lane + 64 * blk;
        const uint32_t off = uint32_t(min(pc / PR, last)) * rs + uint32_t(pc % PR) * 16;
        g2lds16(a.k + row0, off, &sm.RK[buf][blk * 512]);
        g2lds16(a.alpha + row0, off, &sm.RA[buf][blk * 512]);
        g2lds16(a.omega + row0, off, &sm.RW[buf][blk * 512]);
    }
}

// lane t: r_t and mu / r_t of a chunk with nvalid real tokens into LDS
// (padding tokens: r = 1, no precision increment).  GATE: rbits holds the
// pre-activation z and r_t = r_min + softplus(z).
template <int DK, bool GATE = false>
__device__ __forceinline__ void chain_r_store(Smem<DK>& sm, int c, uint32_t rbits, int nvalid, float mu) {
    const int lane = threadIdx.x & 63;
    const bool ok = lane < nvalid;
    float rz = bf1(bf16_t(rbits));
    if (GATE) rz = kGateRMin + gate_softplus(rz);
    const float rt = ok ? rz : 1.f;
    sm.cr[c & 1][lane] = ok ? mu / rt : 0.f;
    if (lane < L) sm.rr[c % 3][lane] = rt;
}

// Gated form, diagonal variant: 1 / |k_t| of tokens 16 hf + 4f .. + 3 of the
// chain's chunk in buffer `buf`, from its raw k tile (16 lanes per row), by
// formation wave f.  Rows 16..31 of the chain's current chunk are read in the
// first half of an iteration (the chain reads their norms after the mid
// barrier), rows 0..15 of its next chunk after that barrier (the state waves'
// copies of them have landed by then).
template <int DK>
__device__ __forceinline__ void chain_knorm_store(Smem<DK>& sm, int buf, int f, int hf) {
    const int lane = threadIdx.x & 63;
    const int row = 16 * hf + 4 * f + (lane >> 4), part = lane & 15;
    constexpr int PER = DK / 16;  // channels per lane: 8 or 4
    const bf16_t* src = &sm.RK[buf][row * DK + part * PER];
    float s = 0.f;
    if (PER == 8) {
        const u4 x = *reinterpret_cast<const u4*>(src);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x0 = bf_lo(x[e]), x1 = bf_hi(x[e]);
            s = fmaf(x0, x0, s);
            s = fmaf(x1, x1, s);
        }
    } else {
        const u2 x = *reinterpret_cast<const u2*>(src);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float x0 = bf_lo(x[e]), x1 = bf_hi(x[e]);
            s = fmaf(x0, x0, s);
            s = fmaf(x1, x1, s);
        }
    }
    s = sum16(s);
    if (part == 0) sm.ks[buf][row] = inv_norm(s);
}

// r_t of chunk c for lane t (lanes >= L repeat the chunk's last token).
// GR: grouped observation noise, r [.., ntile] with one entry per group of
// DVT value columns; this workgroup's columns are group `tile`
template <bool GR>
__device__ __forceinline__ uint32_t chain_r_load(const Args& a, size_t b, int h, int c, int nchunks, int tile,
                                                 int ntile) {
    c = min(max(c, 0), nchunks - 1);
    const int lane = threadIdx.x & 63;
    const size_t tok = tokidx(a, b, h, min(c * L + min(lane, L - 1), a.T - 1));
    return a.r[GR ? tok * size_t(ntile) + size_t(tile) : tok];
}

// bf16 -> fp32 by loading the 16 bits into the upper half of a register whose
// lower half is zero: the load is the conversion.  The compiler emits this
// form only for a fresh register with an explicit clear, so the chain's reads
// are issued from inline assembly into loop-carried input registers whose
// lower halves are zero from the start and never written.  All 48 reads of a
// 16-token range (k, alpha, omega) and the wait for them form ONE asm
// statement: the registers are then defined only once the data is there (with
// separate statements the compiler may copy a register before its load has
// landed).
constexpr int CHAIN_SLOTS = 16;  // tokens per chain segment
static_assert(2 * CHAIN_SLOTS == L && CHAIN_SPLIT == CHAIN_SLOTS, "two 16-token chain segments per chunk");
struct ChainIn {
    uint32_t x[3 * CHAIN_SLOTS];  // k, alpha, omega of the segment's 16 tokens
};
#define KDN_LDH(d, o) "ds_read_u16_d16_hi %" #d ", %48 offset:%" #o "\n\t"
#define KDN_LDH8(d0, d1, d2, d3, d4, d5, d6, d7, o0, o1, o2, o3, o4, o5, o6, o7) \
    KDN_LDH(d0, o0) KDN_LDH(d1, o1) KDN_LDH(d2, o2) KDN_LDH(d3, o3) KDN_LDH(d4, o4) KDN_LDH(d5, o5) \
    KDN_LDH(d6, o6) KDN_LDH(d7, o7)
#define KDN_OUT8(b) \
    "+v"(in.x[b]), "+v"(in.x[b + 1]), "+v"(in.x[b + 2]), "+v"(in.x[b + 3]), "+v"(in.x[b + 4]), \
        "+v"(in.x[b + 5]), "+v"(in.x[b + 6]), "+v"(in.x[b + 7])
#define KDN_IMM16(base)                                                                                     \
    "i"(base), "i"(base + RS), "i"(base + 2 * RS), "i"(base + 3 * RS), "i"(base + 4 * RS), "i"(base + 5 * RS), \
        "i"(base + 6 * RS), "i"(base + 7 * RS), "i"(base + 8 * RS), "i"(base + 9 * RS), "i"(base + 10 * RS),   \
        "i"(base + 11 * RS), "i"(base + 12 * RS), "i"(base + 13 * RS), "i"(base + 14 * RS), "i"(base + 15 * RS)
// in.x[16 m + j] <- tile m (k, alpha, omega) row T0 + j of buffer BUF, for the
// lane address `addr` of column i in the first tile
template <int DK, int BUF, int T0>
__device__ __forceinline__ void chain_read16(ChainIn& in, uint32_t addr) {
    constexpr int TILE = 2 * L * DK * 2;  // bytes of one raw tile pair (two buffers)
    constexpr int RS = DK * 2;            // bytes per row
    constexpr int K0 = BUF * L * DK * 2 + T0 * RS, A0 = TILE + K0, W0 = 2 * TILE + K0;
    static_assert(W0 + 15 * RS < 65536, "LDS immediate offset");
    asm volatile(KDN_LDH8(0, 1, 2, 3, 4, 5, 6, 7, 49, 50, 51, 52, 53, 54, 55, 56)
                 KDN_LDH8(8, 9, 10, 11, 12, 13, 14, 15, 57, 58, 59, 60, 61, 62, 63, 64)
                 KDN_LDH8(16, 17, 18, 19, 20, 21, 22, 23, 65, 66, 67, 68, 69, 70, 71, 72)
                 KDN_LDH8(24, 25, 26, 27, 28, 29, 30, 31, 73, 74, 75, 76, 77, 78, 79, 80)
                 KDN_LDH8(32, 33, 34, 35, 36, 37, 38, 39, 81, 82, 83, 84, 85, 86, 87, 88)
                 KDN_LDH8(40, 41, 42, 43, 44, 45, 46, 47, 89, 90, 91, 92, 93, 94, 95, 96)
                 "s_waitcnt lgkmcnt(0)"
                 : KDN_OUT8(0), KDN_OUT8(8), KDN_OUT8(16), KDN_OUT8(24), KDN_OUT8(32), KDN_OUT8(40)
                 : "v"(addr), KDN_IMM16(K0), KDN_IMM16(A0), KDN_IMM16(W0)
                 : "memory");
}
#undef KDN_LDH
#undef KDN_LDH8
#undef KDN_OUT8
#undef KDN_IMM16

// tokens [T0, T1) of chunk buffer BUF (and KhQ slot gring) with nvalid real
// tokens; p carries across chunks.  g restarts at each half: the first half
// (T0 = 0) forms g_t from the chunk start and stores g_15; the second forms
// gb_t = prod_{16<=u<=t} alpha_u and stores gb_31.  Kh = kappa' / rho: in the
// first half kappa' times the reverse product prod_{t<u<=15} alpha_u (no
// reciprocal), in the second kappa' / gb_t.  Padding tokens (t >= nvalid) act
// as alpha = 1, omega = 0, k = 0: they leave p and g unchanged and write zero
// gain.
template <int DK, int BUF, int T0, int T1, bool MASK, bool GATE>
__device__ __forceinline__ void chain_diag_run(Smem<DK>& sm, ChainIn& in, int i, float& p, float& g, float& gi,
                                               int nvalid, int gring) {
    constexpr int buf = BUF;  // compile-time, so every LDS offset below is an immediate
    constexpr int NTOK = T1 - T0;
    constexpr bool FIRST = T0 == 0;
    static_assert(NTOK == CHAIN_SLOTS, "one 16-token chain segment");
    // read phase: every LDS read of the token range is issued before the
    // recurrence starts (two waves per SIMD cannot hide LDS latency).  The raw
    // tiles sit at the start of the LDS block: one lane address, immediate
    // offsets for the three tiles, both buffers and every row.
    static_assert(offsetof(Smem<DK>, RK) == 0 && offsetof(Smem<DK>, RA) == 2 * L * DK * 2 &&
                      offsetof(Smem<DK>, RW) == 4 * L * DK * 2,
                  "raw chain tiles must be contiguous at the start of the LDS block");
    float cv[NTOK];
#pragma unroll
    for (int j = 0; j < NTOK; ++j) cv[j] = sm.cr[buf][T0 + j];  // same address on every lane: broadcast
    float kn[GATE ? NTOK : 1];  // gated: 1 / |k_t| (the prologue's normalisation of k)
    if (GATE)
#pragma unroll
        for (int j = 0; j < NTOK; j += 4) {
            const f4 x = *reinterpret_cast<const f4*>(&sm.ks[buf][T0 + j]);
#pragma unroll
            for (int e = 0; e < 4; ++e) kn[j + e] = x[e];
        }
    chain_read16<DK, BUF, T0>(in, uint32_t(reinterpret_cast<uintptr_t>((lds_void_t*)&sm.RK[0][i])));
    float kk[NTOK], al[NTOK], w[NTOK], khv[NTOK], gv[NTOK];
    float ez[NTOK];                        // GATE: e^-z of the decay's pre-activation
    uint32_t khp[NTOK / 2], gp[NTOK / 2];  // bf16 pairs of consecutive tokens
#pragma unroll
    for (int j = 0; j < NTOK; ++j) {
        kk[j] = __uint_as_float(in.x[j]);
        al[j] = __uint_as_float(in.x[CHAIN_SLOTS + j]);
        w[j] = __uint_as_float(in.x[2 * CHAIN_SLOTS + j]);
        if (GATE) {
            kk[j] *= kn[j];
            // the decay alpha = 1 / (1 + e^-z) and the process noise from
            // their pre-activations; e^-z is kept for 1 / g below
            ez[j] = __builtin_amdgcn_exp2f(-kLog2E * al[j]);
            al[j] = __builtin_amdgcn_rcpf(1.f + ez[j]);
            w[j] = gate_softplus(w[j]);
        }
        if (MASK) {
            const bool ok = T0 + j < nvalid;
            kk[j] = ok ? kk[j] : 0.f;
            al[j] = ok ? al[j] : 1.f;
            w[j] = ok ? w[j] : 0.f;
            if (GATE) ez[j] = ok ? ez[j] : 0.f;
        }
    }
    // first half: hr[j] = prod_{j<u<16} alpha_u (independent of p, so these
    // multiplies fill the recurrence's dependency gaps)
    float hr[NTOK];
    if (FIRST) {
        hr[NTOK - 1] = 1.f;
#pragma unroll
        for (int j = NTOK - 2; j >= 0; --j) hr[j] = hr[j + 1] * al[j + 1];
    }
#pragma unroll
    for (int j = 0; j < NTOK; ++j) {
        const int t = T0 + j;
        const float asq = al[j] * al[j];
        // the fewest instructions, rather than the shortest dependent path,
        // is what makes this loop fast (one wave per SIMD issues it)
        const float ck = cv[j] * kk[j];           // (mu / r) k
        const float ph = fma3(asq, p, w[j]);      // the only loop-carried chain: ph -> p
        const float kph = kk[j] * ph;             // kappa' = p_hat k
        p = ph * __builtin_amdgcn_rcpf(fmaf(ck, kph, 1.f));  // 1 + (mu / r) k^2 p_hat
        g *= al[j];
        // the gain in the chunk's midpoint frame, kappa'_t / rho_t, and the
        // decay (g_t or gb_t), as bf16 pairs of consecutive tokens.  Both go
        // out in token groups, one wide store per group (a store per token
        // and value would make LDS stores a third of this loop's
        // instructions): the decay in groups of 8 tokens, kappa' / rho as
        // Kh^T in the state's operand order, where the 8 positions of group
        // P / 8 hold tokens 4 (P / 8) + 0..3 and 16 + 4 (P / 8) + 0..3, i.e.
        // a 16-token segment fills one half of each of the four groups.
        if (FIRST) {
            khv[j] = kph * hr[j];
        } else if (GATE) {
            gi = fmaf(gi, ez[j], gi);  // 1 / gb as the product of the (1 + e^-z): no reciprocal
            khv[j] = kph * gi;
        } else {
            khv[j] = kph * __builtin_amdgcn_rcpf(g);
        }
        gv[j] = g;
        if (j & 1) {
            khp[j / 2] = pack2_opaque(khv[j - 1], khv[j]);
            gp[j / 2] = pack2_opaque(gv[j - 1], gv[j]);
        }
        if ((j & 3) == 3)
            *reinterpret_cast<u2*>(&sm.KhQ[gring][((j / 4) * DK + i) * 8 + 4 * (T0 / 16)]) =
                u2{khp[j / 2 - 1], khp[j / 2]};
        if ((j & 7) == 7)
            *reinterpret_cast<u4*>(&sm.GQ[buf][((T0 + j) / 8 * DK + i) * 8]) =
                u4{gp[j / 2 - 3], gp[j / 2 - 2], gp[j / 2 - 1], gp[j / 2]};
        if (t == L / 2 - 1) sm.g15[gring][i] = g;
        if (t == L - 1) sm.gL[gring][i] = g;
    }
}

// Chunk c is outside the chunked form's range when a half-chunk decay (the
// g just formed by a chain) is below kRangeMin on any lane: the first such
// chunk is recorded (every role reads it between barriers).
__device__ __forceinline__ void flag_range(int* bad, float g, int c) {
    if (__any(g < kRangeMin) && (threadIdx.x & 63) == 0) atomicMin(bad, c);
}

// The state carries Sg = diag(g_15) S.  Its per-chunk factor, from chunk c's
// Sg to chunk c + 1's, is f = gb_31(c) g_15(c + 1) (one multiply per
// element).  Where f would fall below the normal fp32 range the state applies
// the two factors one after the other instead; wave w of a chain records that
// for its channels in fsub[slot][w].
template <int DK>
__device__ __forceinline__ void store_fl(Smem<DK>& sm, int slot, int i, float f, int w) {
    sm.fL[slot][i] = f;
    const bool sub = __any(f < 0x1p-124f);
    if ((threadIdx.x & 63) == 0) sm.fsub[slot][w] = sub ? 1 : 0;
}

// ---------------------------------------------------------------------------
// chain role, isotropic variant: lane = token (lanes 32..63 help with |k|^2)
// ---------------------------------------------------------------------------
template <int VAR>
struct ChainIsoRegs {
    u4 kr[8];                       // half a k row (DK/2 channels) of token lane & 31
    u4 ar[VAR == 2 ? 8 : 1];        // per-channel decay: the same half of the alpha row
    bf16_t al, w, rv;               // alpha (scalar decay), omega, r of token lane & 31
};

template <int DK, int VAR>
__device__ __forceinline__ void chain_iso_load(ChainIsoRegs<VAR>& X, const Args& a, size_t b, int h, int c,
                                               int nchunks) {
    c = min(max(c, 0), nchunks - 1);
    const int lane = threadIdx.x & 63;
    const size_t e = tokidx(a, b, h, min(c * L + (lane & 31), a.T - 1));
    constexpr int NQ = DK / 16;  // 16-byte pieces per half row
    const u4* src = reinterpret_cast<const u4*>(a.k + e * DK + (lane >> 5) * (DK / 2));
#pragma unroll
    for (int m = 0; m < NQ; ++m) X.kr[m] = src[m];
    if constexpr (VAR == 2) {
        const u4* asrc = reinterpret_cast<const u4*>(a.alpha + e * DK + (lane >> 5) * (DK / 2));
#pragma unroll
        for (int m = 0; m < NQ; ++m) X.ar[m] = asrc[m];
    } else {
        X.al = a.alpha[e];
    }
    X.w = a.omega[e];
    X.rv = a.r[e];
}

// sum of squares of the bf16 pairs of half a row (lanes 0..31 and 32..63 hold
// the two halves of token lane & 31's row; the result is the whole row's sum)
template <int DK>
__device__ __forceinline__ float row_sumsq(const u4 (&r)[8]) {
    constexpr int NQ = DK / 16;
    float n = 0.f;
#pragma unroll
    for (int m = 0; m < NQ; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x0 = bf_lo(r[m][e]), x1 = bf_hi(r[m][e]);
            n = fmaf(x0, x0, n);
            n = fmaf(x1, x1, n);
        }
    return n + __shfl_xor(n, 32, 64);
}

// the row sums a chunk's scan needs: |k|^2 and (per-channel decay) the
// trace projection mean_i alpha_i^2, of token lane & 31
template <int DK, int VAR, bool GATE = false>
__device__ __forceinline__ void chain_iso_sums(const ChainIsoRegs<VAR>& X, float& n, float& a2) {
    n = row_sumsq<DK>(X.kr);
    if constexpr (VAR == 2) {
        if constexpr (GATE) {
            // the decays from their pre-activations, then mean_i alpha_i^2
            constexpr int NQ = DK / 16;
            float s2 = 0.f;
#pragma unroll
            for (int m = 0; m < NQ; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x0 = gate_sigmoid(bf_lo(X.ar[m][e])), x1 = gate_sigmoid(bf_hi(X.ar[m][e]));
                    s2 = fmaf(x0, x0, s2);
                    s2 = fmaf(x1, x1, s2);
                }
            a2 = (s2 + __shfl_xor(s2, 32, 64)) * (1.f / float(DK));
        } else {
            a2 = row_sumsq<DK>(X.ar) * (1.f / float(DK));
        }
    }
}

template <int DK, int VAR, bool GATE = false>
__device__ __forceinline__ void chain_iso_run(const ChainIsoRegs<VAR>& X, Smem<DK>& sm, int buf, float mu,
                                              float& bprev, int nvalid, int gring, float n, float a2, int c,
                                              float& glprev, bool& flagged) {
    const int lane = threadIdx.x & 63;
    const bool ok = (lane & 31) < nvalid;
    float wz = bf1(bf16_t(X.w)), rz = bf1(bf16_t(X.rv));
    if (GATE) {
        // process and observation noise from their pre-activations
        wz = gate_softplus(wz);
        rz = kGateRMin + gate_softplus(rz);
    }
    const float w = ok ? wz * (1.f / float(DK)) : 0.f;
    const float rt = ok ? rz : 1.f;
    // gated: the prologue's normalisation of k (|k_hat|^2 = |k|^2 / |k|^2;
    // the formation scales its k rows by the same factor)
    const float sk = GATE ? inv_norm(n) : 1.f;
    if (GATE) {
        n *= sk * sk;
        if (lane < L) sm.ks[buf][lane] = sk;
    }
    const float cn = ok ? (mu / (float(DK) * rt)) * n : 0.f;
    // the uncertainty's decay: alpha^2, or with per-channel decay the trace
    // projection mean_i alpha_i^2 (padding tokens: 1)
    float al = 1.f, asq;
    if constexpr (VAR == 2) {
        asq = ok ? a2 : 1.f;
    } else {
        float az = bf1(bf16_t(X.al));
        if (GATE) az = gate_sigmoid(az);
        al = ok ? az : 1.f;
        asq = al * al;
    }
    // this token's Mobius matrix [[m00, m01], [m10, m11]] and decay
    float m00 = asq, m01 = w, m10 = cn * asq, m11 = fmaf(cn, w, 1.f);
    float g = al;
#pragma unroll
    for (int d = 1; d < L; d <<= 1) {
        const float x00 = __shfl_up(m00, d, 32), x01 = __shfl_up(m01, d, 32);
        const float x10 = __shfl_up(m10, d, 32), x11 = __shfl_up(m11, d, 32);
        const float gg = __shfl_up(g, d, 32);
        if ((lane & 31) >= d) {
            // (this block) x (earlier block)
            const float y00 = fmaf(m00, x00, m01 * x10), y01 = fmaf(m00, x01, m01 * x11);
            const float y10 = fmaf(m10, x00, m11 * x10), y11 = fmaf(m10, x01, m11 * x11);
            const float s = __builtin_amdgcn_rcpf(y11);
            m00 = y00 * s;
            m01 = y01 * s;
            m10 = y10 * s;
            m11 = 1.f;
            // the decays restart at token 16, the chunk's midpoint: lanes of
            // the second half take no factor from the first
            if ((lane & 31) < L / 2 || (lane & 31) - d >= L / 2) g *= gg;
        }
    }
    const float bt = (m00 * bprev + m01) / (m10 * bprev + m11);  // b after token t
    float bbefore = __shfl_up(bt, 1, 32);
    if ((lane & 31) == 0) bbefore = bprev;
    if (lane < L) {
        sm.bh[buf][lane] = fmaf(asq, bbefore, w);
        sm.rr[gring][lane] = rt;
    }
    bprev = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bt), L - 1));
    if (VAR == 1) {  // (per-channel decay: the decays come from the decay chain)
        // rho_t = g_t / g_15 in the first half, gb_t in the second
        const float g15 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), L / 2 - 1));
        const float gl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), L - 1));
        if (lane < L) sm.gs[buf][lane] = (lane < L / 2) ? g * __builtin_amdgcn_rcpf(g15) : g;
        // one decay per token: the state reads these three at index 0 (every
        // lane stores the same value there)
        sm.gL[gring][0] = gl;
        sm.g15[gring][0] = g15;
        if (c > 0) {
            const float f = glprev * g15;
            sm.fL[(c - 1) % 3][0] = f;
            sm.fsub[(c - 1) % 3][0] = f < 0x1p-124f ? 1 : 0;
        }
        // the only chain that flags in this variant: the first flag stands
        if ((g15 < kRangeMin || gl < kRangeMin) && !flagged) {
            sm.bad = c;
            flagged = true;
        }
        glprev = gl;
    }
}

// ---------------------------------------------------------------------------
// decay chain (isotropic variant with per-channel decay): lane = channel
// pair (d_k = 128) or channel (64); the cumulative decays g_t,i of a chunk
// ---------------------------------------------------------------------------
template <int DK>
struct DecayRegs {
    uint32_t ap[L];  // alpha of the lane's channel(s) for the chunk's 32 tokens (bf16 pair or value)
};

template <int DK>
__device__ __forceinline__ void chain_decay_load(DecayRegs<DK>& X, const Args& a, size_t b, int h, int c,
                                                 int nchunks) {
    c = min(max(c, 0), nchunks - 1);  // always issue: see the loader note above
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < L; ++t) {
        const size_t e = tokidx(a, b, h, min(c * L + t, a.T - 1)) * DK;
        if (DK == 128) X.ap[t] = reinterpret_cast<const uint32_t*>(a.alpha + e)[lane];
        else X.ap[t] = (a.alpha + e)[lane];
    }
}

// The cumulative decays of the chunk's tokens [T0, T1) (padding tokens:
// alpha = 1): g_t,i = prod_{s <= t} alpha_s,i in the first half, gb_t,i =
// prod_{16 <= s <= t} alpha_s,i in the second (g restarts at 1 between the
// two calls), stored as the diagonal variant's chain stores them (8-token
// groups), g_15 and gb_31 at the ends of the halves; a half-chunk decay below
// the chunked form's range flags chunk c
template <int DK, int T0, int T1, bool MASK, bool GATE = false>
__device__ __forceinline__ void chain_decay_run(const DecayRegs<DK>& X, Smem<DK>& sm, int buf, int nvalid,
                                                int gring, float (&g)[DK / 64], int c, float (&gprev)[DK / 64]) {
    constexpr int CPL = DK / 64;
    const int i0 = CPL * (threadIdx.x & 63);
    float gv[CPL][2];
    uint32_t gp[CPL][4];
#pragma unroll
    for (int t = T0; t < T1; ++t) {
        const bool ok = !MASK || t < nvalid;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            float al = cc ? bf_hi(X.ap[t]) : bf_lo(X.ap[t]);
            if (GATE) al = gate_sigmoid(al);
            g[cc] *= ok ? al : 1.f;
            gv[cc][t & 1] = g[cc];
            if (t & 1) gp[cc][(t >> 1) & 3] = pack2_opaque(gv[cc][0], gv[cc][1]);
            if ((t & 7) == 7)
                *reinterpret_cast<u4*>(&sm.GQ[buf][((t >> 3) * DK + i0 + cc) * 8]) =
                    u4{gp[cc][0], gp[cc][1], gp[cc][2], gp[cc][3]};
        }
    }
    float gmin = g[0], fmin = 1.f;
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
        if (T1 == L) {
            sm.gL[gring][i0 + cc] = g[cc];
            gprev[cc] = g[cc];
        } else {
            sm.g15[gring][i0 + cc] = g[cc];
            if (c > 0) sm.fL[(c - 1) % 3][i0 + cc] = gprev[cc] * g[cc];
            fmin = fminf(fmin, gprev[cc] * g[cc]);
        }
        gmin = fminf(gmin, g[cc]);
    }
    if (T1 != L && c > 0) {
        const bool sub = __any(fmin < 0x1p-124f);
        if ((threadIdx.x & 63) == 0) sm.fsub[(c - 1) % 3][0] = sm.fsub[(c - 1) % 3][1] = sub ? 1 : 0;
    }
    flag_range(&sm.bad, gmin, c);
}

// ---------------------------------------------------------------------------
// formation role: wave f in 0..3 owns tokens [8f, 8f + 8) of a chunk
// ---------------------------------------------------------------------------
template <int DK>
struct FormRegs {
    uint32_t kp[8];  // DK = 128: channels 2l, 2l+1; DK = 64: channel l (low half)
    uint32_t qp[8];
};

template <int DK>
__device__ __forceinline__ void form_load(FormRegs<DK>& X, const Args& a, size_t b, int h, int f, int c,
                                          int nchunks) {
    c = min(max(c, 0), nchunks - 1);  // always issue: see the loader note above
    const unsigned lane = threadIdx.x & 63;
    // token c L + 8 f + tt, clamped to the last one: first row tb, then at
    // most `last` rows further
    const int tb = min(c * L + 8 * f, a.T - 1);
    const int last = min(7, a.T - 1 - tb);
    const size_t e0 = tokidx(a, b, h, tb) * DK;
    const int rs = a.H * DK;  // elements from one token's row to the next
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
        const size_t e = e0 + size_t(min(tt, last) * rs);
        if (DK == 128) {
            X.kp[tt] = reinterpret_cast<const uint32_t*>(a.k + e)[lane];
            X.qp[tt] = reinterpret_cast<const uint32_t*>(a.q + e)[lane];
        } else {
            X.kp[tt] = (a.k + e)[lane];
            X.qp[tt] = (a.q + e)[lane];
        }
    }
}

// 1 / |q_t| (floored norm, the prologue's normalisation) of the formation
// wave's 8 tokens 8f .. 8f + 7 from their bf16 rows in registers (lane l:
// channels CPL l ..) into qs[buf].  Each of the first three exchanges halves
// the set of tokens a lane sums: afterwards lane l holds token
// 4 b5 + 2 b4 + b3 (its bits 5, 4, 3), summed over those three lane bits; a
// sum over the aligned 8-lane group adds the rest.
template <int DK>
__device__ __forceinline__ void form_qnorm_store(Smem<DK>& sm, const uint32_t (&xp)[8], int buf, int f) {
    const int lane = threadIdx.x & 63;
    float v[8];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
        const float x0 = bf_lo(xp[tt]);
        v[tt] = x0 * x0;
        if (DK == 128) {
            const float x1 = bf_hi(xp[tt]);
            v[tt] = fmaf(x1, x1, v[tt]);
        }
    }
    float w4[4], w2[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) w4[j] = halve32(v[j], v[4 + j]);  // bit 5 set: tokens 4..7
#pragma unroll
    for (int j = 0; j < 2; ++j) w2[j] = halve16(w4[j], w4[2 + j]);  // bit 4 set: the upper pair
    // the row rotation by 8 brings lane i the lane whose bit 3 differs: it
    // sends the token this lane keeps
    const bool b3 = lane & 8;
    float w1 = (b3 ? w2[1] : w2[0]) + dpp_mov<kDppRor8>(b3 ? w2[0] : w2[1]);
    w1 = sum8(w1);
    if ((lane & 7) == 0) sm.qs[buf][8 * f + 4 * (lane >> 5) + 2 * ((lane >> 4) & 1) + ((lane >> 3) & 1)] = inv_norm(w1);
}

template <int DK, int VAR, bool MASK, bool GATE = false>
__device__ __forceinline__ void form_run(const FormRegs<DK>& X, Smem<DK>& sm, int nb, int kslot, int f, int nvalid) {
    constexpr bool ISO = VAR != 0;  // one uncertainty scalar per head (Kh formed here)
    const int lane = threadIdx.x & 63;
    constexpr int CPL = DK / 64;           // channels per lane
    const int i0 = CPL * lane;             // first channel of this lane
    const int pos = perm32(i0);            // perm32(i0 + 1) == pos + 1
    // The wave's tokens 8f + 4h + u (h = 0, 1; u = 0..3) are positions
    // u + 4 (f >> 1) of Kh^T group (2f + h) & 3.
    const int hq = 4 * (f >> 1);
    // read phase: the chain's outputs for the wave's 8 tokens
    u4 gq[CPL];     // g of channel i0 + cc, tokens 8f .. 8f + 7 (per-channel decay)
    u2 kq[CPL][2];  // kappa'/g of channel i0 + cc, tokens 8f + 4h .. 8f + 4h + 3 (diagonal variant)
    float gsv[8], bhv[8];  // isotropic scalars: g_t (scalar decay) and b_hat_t
    // gated: the prologue's 1 / |k_t|, stored with the chain's inputs.  (q
    // enters unnormalised: every output term is linear in q_t, so the state
    // scales output row t by 1 / |q_t| instead; this wave forms those below.)
    float skv[GATE ? 8 : 1];
    if (GATE)
#pragma unroll
        for (int j = 0; j < 8; j += 4) {
            const f4 x = *reinterpret_cast<const f4*>(&sm.ks[nb][8 * f + j]);
#pragma unroll
            for (int e = 0; e < 4; ++e) skv[j + e] = x[e];
        }
    if (ISO) {
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
            if (VAR == 1) gsv[tt] = sm.gs[nb][8 * f + tt];
            bhv[tt] = sm.bh[nb][8 * f + tt];
        }
    }
    if (VAR != 1) {
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            gq[cc] = *reinterpret_cast<const u4*>(&sm.GQ[nb][(f * DK + i0 + cc) * 8]);
            if (VAR == 0)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    kq[cc][h] = *reinterpret_cast<const u2*>(
                        &sm.KhQ[kslot][(((2 * f + h) & 3) * DK + i0 + cc) * 8 + hq]);
        }
    }
    // per-channel decays (diagonal and per-channel-decay forms): the chain
    // stores g_t in the first half and gb_t in the second; rho_t is g_t / g_15
    // in the first half (waves f = 0, 1) and gb_t in the second
    float rg[CPL];
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) rg[cc] = (VAR != 1 && f < 2) ? __builtin_amdgcn_rcpf(sm.g15[kslot][i0 + cc]) : 1.f;
    uint32_t kw4[4];  // Kh^T staging (isotropic): the bf16 pairs (DK = 128) or values of 4 tokens
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
        const int t = 8 * f + tt;
        const int off = sw<DK>(t, pos);
        const bool ok = !MASK || t < nvalid;  // tail chunk only: tokens past T read as zero
        const uint32_t kp = ok ? X.kp[tt] : 0u, qp = ok ? X.qp[tt] : 0u;
        float kk[CPL], qq[CPL], g[CPL];
        kk[0] = bf_lo(kp);
        qq[0] = bf_lo(qp);
        if (CPL == 2) {
            kk[CPL - 1] = bf_hi(kp);
            qq[CPL - 1] = bf_hi(qp);
        }
        if (GATE)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) kk[cc] *= skv[tt];
        uint32_t khw;  // this lane's Kh entries of token t
        if (VAR == 1) {
            const float sc = bhv[tt] * __builtin_amdgcn_rcpf(gsv[tt]);
#pragma unroll
            for (int c = 0; c < CPL; ++c) g[c] = gsv[tt];
            khw = CPL == 2 ? pack2(kk[0] * sc, kk[CPL - 1] * sc) : uint32_t(to_bf(kk[0] * sc));
        } else if (VAR == 2) {
            // rho_t per channel from the decay chain; Kh = b_hat_t k / rho_t
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc)
                g[cc] = ((tt & 1) ? bf_hi(gq[cc][tt >> 1]) : bf_lo(gq[cc][tt >> 1])) * rg[cc];
            const float k0 = kk[0] * (bhv[tt] * __builtin_amdgcn_rcpf(g[0]));
            khw = CPL == 2 ? pack2(k0, kk[CPL - 1] * (bhv[tt] * __builtin_amdgcn_rcpf(g[CPL - 1])))
                           : uint32_t(to_bf(k0));
        } else {
            // kappa'_t / rho_t and rho_t from the chain's grouped stores
            const int h = tt >> 2, u = tt & 3;
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc)
                g[cc] = ((tt & 1) ? bf_hi(gq[cc][tt >> 1]) : bf_lo(gq[cc][tt >> 1])) * rg[cc];
            if (CPL == 2)
                khw = __builtin_amdgcn_perm(kq[1][h][u >> 1], kq[0][h][u >> 1], (u & 1) ? 0x07060302u : 0x05040100u);
            else
                khw = (u & 1) ? (kq[0][h][u >> 1] >> 16) : (kq[0][h][u >> 1] & 0xffffu);
        }
        if (CPL == 2) *reinterpret_cast<uint32_t*>(&sm.Kh[off]) = khw;
        else sm.Kh[off] = bf16_t(khw);
        if (CPL == 2) {
            *reinterpret_cast<uint32_t*>(&sm.Kn[nb][off]) = pack2(-kk[0] * g[0], -kk[CPL - 1] * g[CPL - 1]);
            *reinterpret_cast<uint32_t*>(&sm.Qt[nb][off]) = pack2(qq[0] * g[0], qq[CPL - 1] * g[CPL - 1]);
        } else {
            sm.Kn[nb][off] = to_bf(-kk[0] * g[0]);
            sm.Qt[nb][off] = to_bf(qq[0] * g[0]);
        }
        kw4[tt & 3] = khw;
        if (ISO && (tt & 3) == 3) {
            // Kh^T rows i0 (and i0 + 1): the wave's 4 tokens 8f + 4h .. + 3
            // are positions hq .. hq + 3 of group (2f + h) & 3 (the chain
            // writes these in the diagonal variant)
            const int q = ((2 * f + (tt >> 2)) & 3) * DK;
            if (CPL == 2) {
                // byte selectors: low halves of two pairs, high halves of two pairs
                const uint32_t lo01 = __builtin_amdgcn_perm(kw4[1], kw4[0], 0x05040100u);
                const uint32_t lo23 = __builtin_amdgcn_perm(kw4[3], kw4[2], 0x05040100u);
                const uint32_t hi01 = __builtin_amdgcn_perm(kw4[1], kw4[0], 0x07060302u);
                const uint32_t hi23 = __builtin_amdgcn_perm(kw4[3], kw4[2], 0x07060302u);
                *reinterpret_cast<u2*>(&sm.KhQ[kslot][(q + i0) * 8 + hq]) = u2{lo01, lo23};
                *reinterpret_cast<u2*>(&sm.KhQ[kslot][(q + i0 + 1) * 8 + hq]) = u2{hi01, hi23};
            } else {
                *reinterpret_cast<u2*>(&sm.KhQ[kslot][(q + i0) * 8 + hq]) =
                    u2{(kw4[0] & 0xffffu) | (kw4[1] << 16), (kw4[2] & 0xffffu) | (kw4[3] << 16)};
            }
        }
    }
    if (GATE) form_qnorm_store<DK>(sm, X.qp, nb, f);
}

// M, tril(Qt Kh^T) and the diagonal-block inverses of chunk buffer nb; the
// work is split over the four formation waves f
template <int DK>
__device__ __forceinline__ void mphase(Smem<DK>& sm, int nb, int rslot, int f) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int g4 = (lane >> 4) * 4;
    const int kg8 = (lane >> 4) * 8;
    constexpr int KS = DK / 32;
    auto tile = [&](const bf16_t* A, int ra, int rb) {
        b8 av[KS], bv[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            av[kk] = *reinterpret_cast<const b8*>(A + sw<DK>(ra + n, 32 * kk + kg8));
            bv[kk] = *reinterpret_cast<const b8*>(sm.Kh + sw<DK>(rb + n, 32 * kk + kg8));
        }
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) acc = mfma32(av[kk], bv[kk], acc);
        return acc;  // acc[e] = row ra + g4 + e, column rb + n
    };
    if (f == 0) {
        // the diagonal blocks of M = diag(r) + tril(Kt Kh^T) (Kn holds -Kt),
        // column-major fp32, then their inverses
#pragma unroll
        for (int a = 0; a < NT; ++a) {
            const f4 acc = tile(sm.Kn[nb], 16 * a, 16 * a);
            // r of rows g4 .. g4 + 3, read by every lane (a read under the
            // diagonal's select would become a branch and a wait per element)
            const f4 rv = *reinterpret_cast<const f4*>(&sm.rr[rslot][16 * a + g4]);
            f4 mv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tl = g4 + e;
                mv[e] = tl > n ? -acc[e] : (tl == n ? rv[e] - acc[e] : 0.f);
            }
            *reinterpret_cast<f4*>(&sm.Md[a * 256 + n * 16 + g4]) = mv;  // column-major
        }
        wave_lds_sync();
        block_inverse(sm.Md, sm.Wi, sm.Td[nb], lane);
    } else if (f == 1) {
        // block (1,0) of M is -acc: store -M_10 = acc for the substitution;
        // diagonal block (0,0) of tril(Qt Kh^T)
        const f4 acc = tile(sm.Kn[nb], 16, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.Mo[nb][(g4 + e) * 16 + n] = to_bf(acc[e]);
        const f4 q0 = tile(sm.Qt[nb], 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.QK[nb][(g4 + e) * PT + perm32(n)] = to_bf(g4 + e >= n ? q0[e] : 0.f);
    } else if (f == 2) {
        // blocks (1,0) and (1,1) of tril(Qt Kh^T)
        const f4 q10 = tile(sm.Qt[nb], 16, 0);
        const f4 q11 = tile(sm.Qt[nb], 16, 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sm.QK[nb][(16 + g4 + e) * PT + perm32(n)] = to_bf(q10[e]);
            sm.QK[nb][(16 + g4 + e) * PT + perm32(16 + n)] = to_bf(g4 + e >= n ? q11[e] : 0.f);
        }
    }
}

// ---------------------------------------------------------------------------
// state role: wave cw in {0,1} owns 16 NCT value columns, S in registers
// ---------------------------------------------------------------------------
// The state wave's v tile (L tokens x its 16 NCT columns) of chunk c goes to
// LDS ring slot c % 3 by direct loads, two chunks ahead: 64 NCT 16-byte
// pieces, NCT instructions per wave.
template <int DK, int NCT>
__device__ __forceinline__ void state_issue_t(Smem<DK>& sm, const Args& a, size_t b, int h, int colb, int cw,
                                              int c, int nchunks) {
    c = min(max(c, 0), nchunks - 1);  // always exactly NCT instructions (the wait below counts them)
    const int lane = threadIdx.x & 63;
    const int last = a.T - 1 - c * L;
    const bf16_t* base = a.v + tokidx(a, b, h, c * L) * a.DV + colb;
    const uint32_t rs = uint32_t(a.H) * uint32_t(a.DV) * 2;
    constexpr int PPT = 2 * NCT;  // 16-byte pieces per token
#pragma unroll
    for (int m = 0; m < NCT; ++m) {
        const int pc = lane + 64 * m;  // piece: token pc / PPT, columns 8 (pc % PPT) ..
        const uint32_t off = uint32_t(min(pc / PPT, last)) * rs + uint32_t(pc % PPT) * 16;
        g2lds16(base, off, &sm.RV[c % 3][cw][m * 512]);
    }
}

template <int DK, int NCT>
struct StateAcc {
    f4 S[DK / 16][NCT];
    b8 Sb[DK / 32][NCT];  // S as bf16 MFMA operands (rebuilt after each update)
    f4 O[NT][NCT];
    b8 Db[NCT];  // Dn of the chunk (bf16, B-operand layout), per 16-column tile
};
template <int DK, int NCT>
__device__ __forceinline__ void pack_state(StateAcc<DK, NCT>& st) {
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) st.Sb[kk][ct] = pack8(st.S[2 * kk][ct], st.S[2 * kk + 1][ct]);
}

template <int DK, int NCT>
// Rows of a tail chunk past the sequence end need no masking here: their v
// rows repeat the last token (finite), their Kt and Kh are zero, so their Dn
// reaches neither S nor any stored output row.
// S holds Sg = diag(g_15) S_c of this chunk (fp32), Sb its bf16 operands.
__device__ __forceinline__ void state_seg1(StateAcc<DK, NCT>& st, Smem<DK>& sm, int b, int cw, int vslot) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = (lane >> 4) * 4, kg8 = (lane >> 4) * 8;
    constexpr int KS = DK / 32;
    // read phase: v and every A operand of the segment
    uint32_t vr[NT][NCT][4];
    b8 ak[NT][KS], aq[NT][KS];
#pragma unroll
    for (int at = 0; at < NT; ++at) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) vr[at][ct][e] = sm.RV[vslot][cw][(16 * at + g4 + e) * (16 * NCT) + 16 * ct + n];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            ak[at][kk] = *reinterpret_cast<const b8*>(sm.Kn[b] + sw<DK>(16 * at + n, 32 * kk + kg8));
            aq[at][kk] = *reinterpret_cast<const b8*>(sm.Qt[b] + sw<DK>(16 * at + n, 32 * kk + kg8));
        }
    }
    const s4 t0 = *reinterpret_cast<const s4*>(&sm.Td[b][n * 16 + g4]);
    const s4 t1 = *reinterpret_cast<const s4*>(&sm.Td[b][256 + n * 16 + g4]);
    const s4 mo = *reinterpret_cast<const s4*>(&sm.Mo[b][n * 16 + g4]);
    const b8 (&Sb)[KS][NCT] = st.Sb;
    f4 R[NT][NCT];
#pragma unroll
    for (int at = 0; at < NT; ++at) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = bf1(bf16_t(vr[at][ct][e]));
            f4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                r = mfma32(ak[at][kk], Sb[kk][ct], r);  // V - Kt S
                o = mfma32(Sb[kk][ct], aq[at][kk], o);  // (Qt S)^T: value column x token
            }
            R[at][ct] = r;
            st.O[at][ct] = o;
        }
    }
    // Dn = M^-1 R by block substitution (the inverses and -M_10 are ready
    // since the previous iteration)
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const f4 d0 = mfma16(t0, pack4(R[0][ct]), zero);
        const f4 r1 = mfma16(mo, pack4(d0), R[1][ct]);
        const f4 d1 = mfma16(t1, pack4(r1), zero);
        st.Db[ct] = pack8(d0, d1);
    }
}

// S <- diag(g_15) S with g_15 of the chunk in ring slot `slot`
// (SC: one decay per token, the factor sits at index 0)
template <int DK, int NCT, bool SC>
__device__ __forceinline__ void state_scale(StateAcc<DK, NCT>& st, Smem<DK>& sm, int slot) {
    const int g4 = ((threadIdx.x & 63) >> 4) * 4;
    const float g0 = SC ? sm.g15[slot][0] : 0.f;
#pragma unroll
    for (int it = 0; it < DK / 16; ++it) {
        const f4 gh = SC ? f4{g0, g0, g0, g0} : *reinterpret_cast<const f4*>(&sm.g15[slot][16 * it + g4]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) st.S[it][ct][e] *= gh[e];
    }
}

// The update's factor (mode): 0 gb_31 (S itself leaves: the last chunk, or
// the next one is outside the chunked form's range), 1 fL (the next chunk's
// Sg in one multiply), 2 gb_31 then g_15 of the next chunk (fL would leave
// the normal fp32 range).  SC: one decay per token, factors at index 0.
template <int DK, int NCT, bool SC, bool GATE, bool STORE = false>
__device__ __forceinline__ void state_seg2(StateAcc<DK, NCT>& st, Smem<DK>& sm, int b, const Args& a, size_t bb,
                                           int h, int colb, int c, int mode) {
    const int gring = c % 3;
    const bool full = (c + 1) * L <= a.T;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = (lane >> 4) * 4, kg8 = (lane >> 4) * 8;
    // read phase: every LDS operand of the segment
    b8 aqk[NT], akh[DK / 16];
    f4 glv[DK / 16];
#pragma unroll
    for (int at = 0; at < NT; ++at) aqk[at] = *reinterpret_cast<const b8*>(&sm.QK[b][(16 * at + n) * PT + kg8]);
#pragma unroll
    for (int it = 0; it < DK / 16; ++it) {
        akh[it] = *reinterpret_cast<const b8*>(&sm.KhQ[gring][((lane >> 4) * DK + 16 * it + n) * 8]);
        if (!SC) glv[it] = *reinterpret_cast<const f4*>(mode == 1 ? &sm.fL[gring][16 * it + g4] : &sm.gL[gring][16 * it + g4]);
    }
    if (SC) {
        const float g0 = mode == 1 ? sm.fL[gring][0] : sm.gL[gring][0];
#pragma unroll
        for (int it = 0; it < DK / 16; ++it) glv[it] = f4{g0, g0, g0, g0};
    }
    const b8* Db = st.Db;
    // outputs, transposed: lane (n, g4) holds value columns g4 .. g4 + 3 of
    // token 16 at + n, written as one 8-byte store per tile
    bf16_t* orow = a.o + tokidx(a, bb, h, c * L + n) * a.DV + colb + g4;
    const size_t ostep = size_t(16) * a.H * a.DV;  // 16 tokens
#pragma unroll
    for (int at = 0; at < NT; ++at) {
        const bool ok = full || c * L + 16 * at + n < a.T;
        const float sq = GATE ? sm.qs[b][16 * at + n] : 1.f;  // gated: the prologue's 1 / |q_t|
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f4 o = mfma32(Db[ct], aqk[at], st.O[at][ct]);  // (tril(Qt Kh^T) Dn)^T
            if (GATE) o *= sq;
            if (ok && !STORE) *reinterpret_cast<u2*>(orow + 16 * ct) = u2{pack2(o[0], o[1]), pack2(o[2], o[3])};
        }
        orow += ostep;
    }
    // S <- diag(gb_31) (Sg + Kh^T Dn), and the next chunk's Sg
#pragma unroll
    for (int it = 0; it < DK / 16; ++it) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f4 s = mfma32(akh[it], Db[ct], st.S[it][ct]);
#pragma unroll
            for (int e = 0; e < 4; ++e) s[e] *= glv[it][e];
            st.S[it][ct] = s;
        }
    }
    if (mode == 2) state_scale<DK, NCT, SC>(st, sm, (c + 1) % 3);
    pack_state<DK, NCT>(st);  // operands of the next chunk's first segment
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
// Wave w of the workgroup runs on SIMD w % 4.  Waves 0 and 1 run the chain;
// ROLE_LAYOUT places the two state waves and the four formation waves
// (formation index f = 0..3) on the SIMDs:
//   0: state 4, 5;  formation 2, 3, 6, 7
//   1: state 6, 7;  formation 2, 3, 4, 5
//   2: state 6, 7;  formation 4, 5, 2, 3
constexpr int ROLE_LAYOUT = 0;
__device__ __forceinline__ bool is_state_wave(int w) {
    return ROLE_LAYOUT == 0 ? (w == 4 || w == 5) : (w == 6 || w == 7);
}
__device__ __forceinline__ int state_index(int w) { return ROLE_LAYOUT == 0 ? w - 4 : w - 6; }
__device__ __forceinline__ int form_index(int w) {
    return ROLE_LAYOUT == 0 ? (w < 4 ? w - 2 : w - 4) : ROLE_LAYOUT == 1 ? w - 2 : (w >= 4 ? w - 4 : w);
}
// VAR: 0 diagonal, 1 isotropic, 2 isotropic with per-channel decay.
// GR (diagonal only): grouped observation noise, one r and one uncertainty
// state p per group of DVT value columns, i.e. per column tile; the tiles of
// a head are then independent diagonal recurrences sharing q, k, alpha, omega.
template <int DK, int VAR, bool GR = false, int NCT = 2, bool GATE = false, bool STORE = false>
__global__ void __launch_bounds__(NTHREADS) kdn_chunk_kernel(Args a) {
    constexpr bool ISO = VAR != 0;  // one uncertainty scalar per head
    static_assert(!GATE || !GR, "no gate step with grouped observation noise");
    static_assert(!STORE || (VAR == 0 && !GR && NCT == 2), "checkpoints: diagonal, 64-column tiles");
    static_assert(!GR || VAR == 0, "grouped noise is a diagonal form");
    static_assert(!GR || NCT == 2, "a noise group is one 64-column tile");
    constexpr int DVTN = dvt_of<NCT>();  // value columns of this workgroup
    __shared__ Smem<DK> sm;
    const int ntile = a.seg ? a.vtiles + DK / DVTN : a.DV / DVTN;
    const int bid = blockIdx.x;
    // Work items are dealt to the eight XCDs in turn (block bid runs on XCD
    // bid % 8); the column tiles of one (batch, head) pair share an XCD and
    // its L2.  Items are numbered batch-fastest, so with B a multiple of 8
    // an XCD streams whole [H, d] token rows of its batches rather than a
    // fixed slice of every row (which would keep hitting the same HBM
    // channels).
    const int item = (bid / (8 * ntile)) * 8 + (bid % 8);
    const int tile = (bid / 8) % ntile;
    if (item >= a.units) return;
    const int nbatch = a.units / a.H;
    int h = item / nbatch;  // [B,T,H] batch: items batch-fastest (above)
    size_t b = size_t(item % nbatch);
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int lane = threadIdx.x & 63;
    // this item's sequence: a.T tokens from grid row a.tok0 on.  Packed
    // sequences of different lengths are numbered head-fastest in their
    // scheduling order (all heads of the first sequence of a.ord first):
    // blocks start roughly in this order as CUs free up, so with the longest
    // sequences first the work spreads evenly over the CUs.  Their bounds
    // come from the offsets, clamped into the grid (a.T is then the grid's
    // token count), so no offset can reach outside it.
    int seg_g = 0;     // segment mode: this workgroup's segment
    bool phi = false;  // segment mode: a tile of the identity columns
    if (a.seg) {
        const int nunit = a.units / a.nseg;  // (batch, head) pairs
        seg_g = item / nunit;
        const int u = item % nunit;
        b = size_t(u / a.H);
        h = u % a.H;
        const int total = a.T;
        const int s0 = seg_g * a.seg;
        a.tok0 = b * size_t(total) + size_t(s0);
        a.T = min(a.seg, total - s0);
        phi = tile >= a.vtiles;
        if (phi && seg_g == 0) return;  // the first segment starts from S0 itself
    } else if (a.cu) {
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
    const int unit = int(b) * a.H + h;  // (batch, head) index of the [B, H, ...] states
    if (a.T == 0) {
        // an empty sequence: the final state is the initial one
        const size_t sb = size_t(unit) * DK * a.DV;
        for (int e = threadIdx.x; e < DK * DVTN; e += NTHREADS) {
            const size_t x = sb + size_t(e / DVTN) * a.DV + tile * DVTN + e % DVTN;
            a.S_T[x] = a.S0 ? a.S0[x] : 0.f;
        }
        if (GR || tile == 0) {
            const int np = ISO ? 1 : DK;
            const size_t pb = GR ? (size_t(unit) * ntile + tile) * np : size_t(unit) * np;
            for (int i = threadIdx.x; i < np; i += NTHREADS) a.p_T[pb + i] = a.p0 ? a.p0[pb + i] : a.c0[h];
        }
        return;
    }
    const int nchunks = (a.T + L - 1) / L;
    const int nit = ((nchunks + 2) + 1) & ~1;  // even number of pipeline iterations

    // the chain's first input tiles (issued by the formation waves)
    const bool is_form = wave >= 2 && !is_state_wave(wave);
    const int fwave = form_index(wave);
    uint32_t r0 = 0;
    if (VAR == 0 && is_form) {
        chain_diag_issue<DK, 0, 4>(sm, a, b, h, 0, nchunks, fwave);
        chain_diag_issue<DK, 1, 4>(sm, a, b, h, 0, nchunks, fwave);
        chain_diag_issue<DK, 0, 4>(sm, a, b, h, 1, nchunks, fwave);
        if (fwave == 3) r0 = chain_r_load<GR>(a, b, h, 0, nchunks, tile, ntile);
    }
    // rows 0..15 of tril(Qt Kh^T) never touch tokens 16..31, and the block
    // (0,1) of each diagonal-block inverse is zero: write both once
    for (int e = threadIdx.x; e < 2 * 16 * 16; e += NTHREADS) {
        const int bb = e >> 8, t = (e >> 4) & 15, s = 16 + (e & 15);
        sm.QK[bb][t * PT + perm32(s)] = 0;
        const int a = (e >> 6) & 1, tt = (e >> 3) & 7, ss = 8 + (e & 7);
        sm.Td[bb][a * 256 + tt * 16 + ss] = 0;
    }
    if (threadIdx.x == 0) sm.bad = INT_MAX;
    if (threadIdx.x < 6) sm.fsub[threadIdx.x >> 1][threadIdx.x & 1] = 0;
    vm_wait<0>();  // chunk 0's tiles and r have landed
    if (VAR == 0 && is_form && fwave == 3) chain_r_store<DK, GATE>(sm, 0, r0, min(L, a.T), a.mu);
    if (GATE && VAR == 0) {
        bar();  // every wave's copies of chunk 0's k rows have landed
        if (is_form) chain_knorm_store<DK>(sm, 0, fwave, 0);  // rows 16..31: in the loop
    }
    bar();

    // Range flags.  A chain flags chunk c (sm.bad, the smallest such c)
    // during iteration c when a half-chunk decay leaves the chunked form's
    // range.  The roles still run every iteration (the chunks from bad on
    // compute values nobody stores); the state waves skip chunks from bad on,
    // so their S stays the state at chunk bad's start, and the chains keep the
    // uncertainty at that start.  After the loop every wave reads the same
    // sm.bad; if it is set, the workgroup finishes the sequence with the token
    // recurrence from chunk bad on (below).
    int bad_seen = INT_MAX;
    // chain: the uncertainty at the start of the last two chunks, and at the
    // start of the first flagged chunk (diagonal: per lane)
    float pst[2] = {0.f, 0.f}, psave = 0.f;
    if (wave == 0 || wave == 1) {
        // ---------------- chain ----------------
        if (VAR == 0) {
            const bool active = wave < DK / 64;
            const int i = wave * 64 + lane;
            float p = 0.f;
            const size_t pidx = (GR ? size_t(unit) * ntile + tile : size_t(unit)) * DK + i;
            if (active) {
                p = a.p0 ? a.p0[pidx] : a.c0[h];
                // segment mode: the uncertainty at the segment's start, the
                // preceding segments' Mobius maps applied to p0 in order
                for (int gg = 0; gg < seg_g; ++gg) {
                    const float4 m = *reinterpret_cast<const float4*>(
                        a.mob + ((size_t(unit) * a.nseg + gg) * DK + i) * 4);
                    p = (m.x * p + m.y) / (m.z * p + m.w);
                }
            }
            settle(p);  // p is ready before the pipelined loop
            // chunk c's tiles are in LDS buffer c & 1 (chunk c + 1's are
            // fetched meanwhile by the formation waves); the loop runs two
            // chunks per trip so that the buffer index is a constant
            ChainIn in;
#pragma unroll
            for (int j = 0; j < 3 * CHAIN_SLOTS; ++j) in.x[j] = 0u;
            float gprev = 1.f;  // gb_31 of the previous chunk
            auto step = [&](auto bufc, int c) {
                constexpr int BUF = decltype(bufc)::value;
                const int nvalid = min(L, a.T - c * L);
                bad_seen = sm.bad;  // flags of chunks before c
                if (bad_seen == c - 1) psave = pst[BUF ^ 1];
                pst[BUF] = p;
                if (STORE && tile == 0 && active && c < nchunks) a.ckp[(size_t(unit) * nchunks + c) * DK + i] = p;
                float g = 1.f, gi = 1.f;
                if (active && c < nchunks) {
                    if (nvalid == L) chain_diag_run<DK, BUF, 0, CHAIN_SPLIT, false, GATE>(sm, in, i, p, g, gi, L, c % 3);
                    else chain_diag_run<DK, BUF, 0, CHAIN_SPLIT, true, GATE>(sm, in, i, p, g, gi, nvalid, c % 3);
                    flag_range(&sm.bad, g, c);
                    if (c > 0) store_fl(sm, (c - 1) % 3, i, gprev * g, wave);
                }
                bar();
                g = 1.f;
                gi = 1.f;
                if (active && c < nchunks) {
                    if (nvalid == L) chain_diag_run<DK, BUF, CHAIN_SPLIT, L, false, GATE>(sm, in, i, p, g, gi, L, c % 3);
                    else chain_diag_run<DK, BUF, CHAIN_SPLIT, L, true, GATE>(sm, in, i, p, g, gi, nvalid, c % 3);
                    flag_range(&sm.bad, g, c);
                    gprev = g;
                }
                bar();
            };
            for (int c = 0; c < nit; c += 2) {
                step(IntC<0>{}, c);
                step(IntC<1>{}, c + 1);
            }
            bad_seen = sm.bad;
            if (!STORE && bad_seen >= nchunks && active && (GR || tile == 0) && seg_g == a.nseg - 1) a.p_T[pidx] = p;
        } else if (wave == 1) {
            // the per-channel decays (isotropic variant with per-channel
            // decay; otherwise this wave only keeps the barrier count)
            DecayRegs<DK> A, B;
            if (VAR == 2) chain_decay_load<DK>(A, a, b, h, 0, nchunks);
            float gprev[DK / 64];
#pragma unroll
            for (int cc = 0; cc < DK / 64; ++cc) gprev[cc] = 1.f;
            for (int it = 0; it < nit; it += 2) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    DecayRegs<DK>& X = half ? B : A;
                    DecayRegs<DK>& Y = half ? A : B;
                    const int c = it + half;
                    // tokens 0..15 of chunk c in the first segment, then the
                    // loads of chunk c + 1 (into the other register set),
                    // tokens 16..31 in the second segment
                    const int nvalid = min(L, a.T - c * L);
                    float g[DK / 64];
#pragma unroll
                    for (int cc = 0; cc < DK / 64; ++cc) g[cc] = 1.f;
                    if (VAR == 2) {
                        if (c < nchunks) {
                            if (nvalid == L) chain_decay_run<DK, 0, L / 2, false, GATE>(X, sm, c & 1, L, c % 3, g, c, gprev);
                            else chain_decay_run<DK, 0, L / 2, true, GATE>(X, sm, c & 1, nvalid, c % 3, g, c, gprev);
                        }
                        chain_decay_load<DK>(Y, a, b, h, c + 1, nchunks);
                    }
                    bar();
#pragma unroll
                    for (int cc = 0; cc < DK / 64; ++cc) g[cc] = 1.f;
                    if (VAR == 2 && c < nchunks) {
                        if (nvalid == L) chain_decay_run<DK, L / 2, L, false, GATE>(X, sm, c & 1, L, c % 3, g, c, gprev);
                        else chain_decay_run<DK, L / 2, L, true, GATE>(X, sm, c & 1, nvalid, c % 3, g, c, gprev);
                    }
                    bar();
                }
            }
            bad_seen = sm.bad;
        } else {
            float bprev = a.p0 ? a.p0[unit] : a.c0[h];
            settle(bprev);
            ChainIsoRegs<VAR> A, B;
            chain_iso_load<DK, VAR>(A, a, b, h, 0, nchunks);
            // the row sums of the next chunk are formed in the second segment
            // (this wave's idle one), from the registers just loaded
            float n = 0.f, a2 = 1.f, glprev = 1.f;
            bool flagged = false;
            chain_iso_sums<DK, VAR, GATE>(A, n, a2);
            for (int it = 0; it < nit; it += 2) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    ChainIsoRegs<VAR>& X = half ? B : A;
                    ChainIsoRegs<VAR>& Y = half ? A : B;
                    const int c = it + half;
                    if (VAR == 2) {
                        bad_seen = sm.bad;  // the decay chain's flags of chunks before c
                        if (bad_seen == c - 1) psave = pst[half ^ 1];
                    } else if (!flagged) {
                        psave = bprev;  // this chain flags: keep the start of the last unflagged chunk
                    }
                    pst[half] = bprev;
                    {
                        // the next chunk's loads go out after this chunk's
                        // registers are consumed: issued earlier, their
                        // address temporaries would be placed in registers of
                        // loads still in flight, and the compiler would wait
                        // for those loads (a full memory round trip) first
                        if (c < nchunks)
                            chain_iso_run<DK, VAR, GATE>(X, sm, c & 1, a.mu, bprev, min(L, a.T - c * L), c % 3, n, a2,
                                                         c, glprev, flagged);
                        chain_iso_load<DK, VAR>(Y, a, b, h, c + 1, nchunks);
                    }
                    bar();
                    chain_iso_sums<DK, VAR, GATE>(Y, n, a2);
                    bar();
                }
            }
            bad_seen = sm.bad;
            if (bad_seen >= nchunks && lane == 0 && tile == 0) a.p_T[unit] = bprev;
        }
    } else if (is_state_wave(wave)) {
        // ---------------- state ----------------
        const int cw = state_index(wave);
        const int colb = tile * DVTN + cw * (16 * NCT);
        const int n = lane & 15, g4 = (lane >> 4) * 4;
        StateAcc<DK, NCT> st;
        const size_t sbase = size_t(unit) * DK * a.DV;
        const bool s0in = a.S0 && seg_g == 0;
#pragma unroll
        for (int it = 0; it < DK / 16; ++it)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * it + g4 + e, col = colb + 16 * ct + n;
                    st.S[it][ct][e] = phi ? (row == col - a.DV ? 1.f : 0.f)
                                          : s0in ? a.S0[sbase + size_t(row) * a.DV + col] : 0.f;
                }
        // identity columns: v = 0 (their v ring holds zeros, never reloaded),
        // o to the identity outputs
        if (phi) {
#pragma unroll
            for (int sl = 0; sl < 3; ++sl)
                for (int x = lane; x < L * 32 / 8; x += 64) *reinterpret_cast<u4*>(&sm.RV[sl][cw][8 * x]) = u4{0u, 0u, 0u, 0u};
        }
        Args ao = a;
        if (phi) {
            ao.o = a.ophi;
            ao.DV = DK;
        }
        const int colo = phi ? colb - a.DV : colb;
#pragma unroll
        for (int it = 0; it < DK / 16; ++it)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) settle(st.S[it][ct]);  // S0 is ready before the loop
        // Chunk it's v is issued at iteration it, waited for at iteration
        // it + 1 and consumed at iteration it + 2 (ring slot it % 3).
        // Iterations 0 and 1 consume nothing; at iteration 1 the chain has
        // stored chunk 0's g_15, and S0 becomes chunk 0's Sg.
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            bad_seen = sm.bad;
            if (!phi) state_issue_t<DK, NCT>(sm, a, b, h, colb, cw, it, nchunks);
            vm_wait<NCT>();
            bar();
            if (VAR == 0) chain_diag_issue<DK, 0, 2>(sm, a, b, h, it + 2, nchunks, cw);
            if (it == 1) {
                if (0 < bad_seen) state_scale<DK, NCT, VAR == 1>(st, sm, 0);
                pack_state<DK, NCT>(st);
            }
            bar();
        }
        for (int it = 2; it < nit; ++it) {
            // Chunks from the first one outside the chunked form's range on
            // are skipped (its flag is visible since iteration c + 1): S then
            // stays the state at that chunk's start.
            const int c = it - 2;  // chunk consumed at this iteration
            bad_seen = sm.bad;
            const int fsub = sm.fsub[c % 3][0] | sm.fsub[c % 3][1];  // read early: its use is a segment away
            const bool run = c < nchunks && c < bad_seen;
            if (!phi) state_issue_t<DK, NCT>(sm, a, b, h, colb, cw, it, nchunks);
            if (run) state_seg1<DK, NCT>(st, sm, c & 1, cw, c % 3);
            // everything but the NCT loads just issued has landed: the v of
            // chunk it - 1, the previous iteration's stores and chain rows
            vm_wait<NCT>();
            if (STORE && run) {
                // chunk c's start state, diag(g_15) S (the first segment leaves
                // it unchanged), rounded to bf16 as [DK / 4][64][4]: rows 4j ..
                // 4j + 3 of a column in one 8-byte store.  Issued after the
                // wait, so that they complete during the next iteration.
                u2* ck = reinterpret_cast<u2*>(a.cks + ((size_t(unit) * ntile + tile) * nchunks + c) * DK * DVTN);
#pragma unroll
                for (int r4 = 0; r4 < DK / 16; ++r4)
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        const f4 x = st.S[r4][ct];
                        ck[((16 * r4 + g4) / 4) * DVTN + cw * (16 * NCT) + 16 * ct + n] = u2{pack2(x[0], x[1]), pack2(x[2], x[3])};
                    }
            }
            bar();
            // rows 0..15 of the chain's chunk it + 2: the chain has read those
            // rows of chunk it (same buffer) before the barrier above
            if (VAR == 0) chain_diag_issue<DK, 0, 2>(sm, a, b, h, it + 2, nchunks, cw);
            if (run) {
                const bool next = c + 1 < nchunks && c + 1 < bad_seen;
                const int mode = !next ? 0 : fsub ? 2 : 1;
                state_seg2<DK, NCT, VAR == 1, GATE, STORE>(st, sm, c & 1, ao, b, h, colo, c, mode);
            }
            bar();
        }
        bad_seen = sm.bad;
        if (STORE) {
            // no final state in checkpoint mode
        } else if (bad_seen >= nchunks) {
            // segment mode: the segment's end state, [v | identity] columns
            float* sout = a.seg ? a.sseg + (size_t(unit) * a.nseg + seg_g) * DK * (a.DV + DK) : a.S_T + sbase;
            const int sstride = a.seg ? a.DV + DK : a.DV;
#pragma unroll
            for (int it = 0; it < DK / 16; ++it)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sout[size_t(16 * it + g4 + e) * sstride + colb + 16 * ct + n] = st.S[it][ct][e];
        } else {
            // hand-off: S_bad of this wave's columns
            vm_wait<0>();
            bar();
            Handoff<DK>& hf = *reinterpret_cast<Handoff<DK>*>(&sm);
#pragma unroll
            for (int it = 0; it < DK / 16; ++it)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        hf.S[16 * it + g4 + e][cw * (16 * NCT) + 16 * ct + n] = st.S[it][ct][e];
        }
    } else {
        // ---------------- formation ----------------
        const int f = fwave;
        FormRegs<DK> A, B;
        // chunk c is formed at iteration c + 1; its q, k are loaded one iteration earlier
        for (int it = 0; it < nit; it += 2) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                FormRegs<DK>& X = half ? B : A;
                FormRegs<DK>& Y = half ? A : B;
                const int c = it + half - 1;
                // the chain's inputs for chunk c + 2 (it consumes chunk c + 1 now)
                uint32_t rnext = 0;
                if (VAR == 0) {
                    chain_diag_issue<DK, 1, 4>(sm, a, b, h, c + 2, nchunks, f);  // rows 16..31
                    if (f == 3) rnext = chain_r_load<GR>(a, b, h, c + 2, nchunks, tile, ntile);
                }
                form_load<DK>(Y, a, b, h, f, c + 1, nchunks);
                if (GATE && VAR == 0 && c + 1 < nchunks) chain_knorm_store<DK>(sm, (c + 1) & 1, f, 1);
                if (c >= 0 && c < nchunks) {
                    const int nvalid = min(L, a.T - c * L);
                    if (nvalid == L) form_run<DK, VAR, false, GATE>(X, sm, c & 1, c % 3, f, L);
                    else form_run<DK, VAR, true, GATE>(X, sm, c & 1, c % 3, f, nvalid);
                }
                bar();
                if (GATE && VAR == 0 && c + 2 < nchunks) chain_knorm_store<DK>(sm, c & 1, f, 0);
                if (c >= 0 && c < nchunks) mphase<DK>(sm, c & 1, c % 3, f);
                // everything issued this iteration has landed: the chain's tiles
                // for chunk c + 2 and q, k of chunk c + 1.  Settling the latter
                // tells the compiler so; otherwise its wait before the next
                // form_run would count the untracked copies and stall on them.
                vm_wait<0>();
#pragma unroll
                for (int tt = 0; tt < 8; ++tt) {
                    settle(Y.kp[tt]);
                    settle(Y.qp[tt]);
                }
                if (VAR == 0) {
                    settle(rnext);
                    if (f == 3) chain_r_store<DK, GATE>(sm, c + 2, rnext, min(L, a.T - (c + 2) * L), a.mu);
                }
                bar();
            }
        }
        bad_seen = sm.bad;
    }
    if (STORE && tile == 0 && threadIdx.x == 0) a.ck_flag[unit] = bad_seen < nchunks ? 1 : 0;
    if (STORE || bad_seen >= nchunks) {
        vm_wait<0>();  // no direct copy may land after the workgroup's LDS is released
        return;
    }

    // ---------------- hand-off to the token recurrence ----------------
    // chunk bad_seen and the rest of the sequence, from the state the chunked
    // form carried to the start of that chunk (the state waves wrote S above)
    Handoff<DK>& hf = *reinterpret_cast<Handoff<DK>*>(&sm);
    if (!is_state_wave(wave)) {
        vm_wait<0>();  // direct copies still in flight land before their LDS is reused
        bar();
        if (wave < 2) {
            if (VAR == 0) {
                if (wave < DK / 64) hf.p[wave * 64 + lane] = psave;
            } else if (wave == 0 && lane == 0) {
                hf.p[0] = psave;
            }
        }
    }
    bar();
    constexpr int NRW = DVTN / 32;  // recurrence waves: 32 value columns each
    if (wave >= NRW) return;
    constexpr int CPL = DK / 64, RPT = DK / 8;
    const int cq = lane & 7, rg = lane >> 3;
    const int lcol = wave * 32 + cq * 4;  // column within the workgroup's tile
    float S[RPT][4], p[CPL], pb = 0.f;
#pragma unroll
    for (int m = 0; m < RPT; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[m][j] = hf.S[rg + 8 * m][lcol + j];
    if (VAR != 0) {
        pb = hf.p[0];
    } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) p[c] = hf.p[lane + 64 * c];
    }
    const int col = tile * DVTN + lcol;  // column within the head ([v | identity] in segment mode)
    // identity columns: v = 0 (not read), outputs to the identity outputs
    const rec::RecIO<bf16_t> io{a.q, a.k, phi ? nullptr : a.v, a.alpha, a.omega, a.r, phi ? a.ophi : a.o, a.mu, a.H,
                                phi ? DK : a.DV, h, a.tok0, phi ? col - a.DV : col, ntile, tile, GATE};
    if (phi) rec::run_tokens<DK, VAR, bf16_t, GR, true>(io, S, p, pb, hf.chan[wave], bad_seen * L, a.T);
    else rec::run_tokens<DK, VAR, bf16_t, GR>(io, S, p, pb, hf.chan[wave], bad_seen * L, a.T);
    float* sout = a.seg ? a.sseg + (size_t(unit) * a.nseg + seg_g) * DK * (a.DV + DK) : a.S_T + size_t(unit) * DK * a.DV;
    const int sstride = a.seg ? a.DV + DK : a.DV;
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        *reinterpret_cast<float4*>(sout + size_t(rg + 8 * m) * sstride + col) =
            make_float4(S[m][0], S[m][1], S[m][2], S[m][3]);
    if (wave == 0 && (GR || tile == 0) && seg_g == a.nseg - 1) {
        if (VAR != 0) {
            if (lane == 0) a.p_T[unit] = pb;
        } else {
            const size_t pb0 = (GR ? size_t(unit) * ntile + tile : size_t(unit)) * DK;
#pragma unroll
            for (int c = 0; c < CPL; ++c) a.p_T[pb0 + lane + 64 * c] = p[c];
        }
    }
}

template <int DK, int VAR, bool GR = false, int NCT = 2, bool GATE = false>
hipError_t launch_t(const FwdArgs& f, hipStream_t stream) {
    const int units = f.B * f.H;
    if (units == 0) return hipSuccess;
    Args a;
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
    const int ntile = f.dv / dvt_of<NCT>();
    const int groups = (units + 7) / 8;
    const unsigned grid = unsigned(groups) * 8u * unsigned(ntile);
    hipLaunchKernelGGL((kdn_chunk_kernel<DK, VAR, GR, NCT, GATE>), dim3(grid), dim3(NTHREADS), 0, stream, a);
    return hipGetLastError();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Segment mode of the diagonal form (64-column tiles): B * H * nseg items,
// each with d_v / 64 tiles of v columns and d_k / 64 tiles of identity columns.
template <int DK>
hipError_t launch_segments_t(const FwdArgs& f, int seg, int nseg, const float* mob, bf16_t* ophi, float* sseg,
                             hipStream_t stream) {
    const int units = f.B * f.H * nseg;
    if (units == 0) return hipSuccess;
    Args a;
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
    a.cu = nullptr;
    a.ord = nullptr;
    a.tok0 = 0;
    a.seg = seg;
    a.nseg = nseg;
    a.vtiles = f.dv / DVT;
    a.mob = mob;
    a.ophi = ophi;
    a.sseg = sseg;
    const int ntile = a.vtiles + DK / DVT;
    const int groups = (units + 7) / 8;
    const unsigned grid = unsigned(groups) * 8u * unsigned(ntile);
    hipLaunchKernelGGL((kdn_chunk_kernel<DK, 0, false, 2, false>), dim3(grid), dim3(NTHREADS), 0, stream, a);
    return hipGetLastError();
}

// Checkpoint sweep of the chunked backward (diagonal, bf16, 64-column tiles;
// GATE: the gated forward's values).
template <int DK, bool GATE>
hipError_t launch_checkpoints_t(const FwdArgs& f, bf16_t* cks, float* ckp, int* ck_flag, hipStream_t stream) {
    const int units = f.B * f.H;
    if (units == 0 || f.T == 0) return hipSuccess;
    Args a;
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
    a.o = nullptr;
    a.S_T = nullptr;
    a.p_T = nullptr;
    a.cu = nullptr;
    a.ord = nullptr;
    a.tok0 = 0;
    a.cks = cks;
    a.ckp = ckp;
    a.ck_flag = ck_flag;
    const int ntile = f.dv / DVT;
    const int groups = (units + 7) / 8;
    const unsigned grid = unsigned(groups) * 8u * unsigned(ntile);
    hipLaunchKernelGGL((kdn_chunk_kernel<DK, 0, false, 2, GATE, true>), dim3(grid), dim3(NTHREADS), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunked_checkpoints(const FwdArgs& a, uint16_t* cks, float* ckp, int* ck_flag,
                                      hipStream_t stream) {
    if (!chunked_supports(a) || a.variant != 0 || a.cu_seqlens) return hipErrorNotSupported;
    if (a.gates)
        return a.dk == 128 ? launch_checkpoints_t<128, true>(a, cks, ckp, ck_flag, stream)
                           : launch_checkpoints_t<64, true>(a, cks, ckp, ck_flag, stream);
    return a.dk == 128 ? launch_checkpoints_t<128, false>(a, cks, ckp, ck_flag, stream)
                       : launch_checkpoints_t<64, false>(a, cks, ckp, ck_flag, stream);
}

// Compute units of the current device (read once per device and cached; 256
// on MI355X).  A failed query gives 256.
long device_cus() {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cache[kMaxDev] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

namespace {

// Narrow workgroups (32 value columns) when the 64-column tiling leaves more
// than half of the device's CUs without a workgroup: one workgroup holds one
// CU (its LDS), and a chunk takes as long in either width, so twice the
// workgroups halve the time while they still fit on the CUs at once.
bool narrow_pays(const FwdArgs& a) {
    if (a.chunk_width != 0) return a.chunk_width == dvt_of<1>();
    return long(a.B) * a.H * (a.dv / DVT) * 2 <= device_cus();
}

template <int DK>
hipError_t launch_gated(const FwdArgs& a, hipStream_t stream) {
    if (narrow_pays(a)) {
        if (a.variant == 2) return launch_t<DK, 2, false, 1, true>(a, stream);
        return launch_t<DK, 0, false, 1, true>(a, stream);
    }
    if (a.variant == 2) return launch_t<DK, 2, false, 2, true>(a, stream);
    return launch_t<DK, 0, false, 2, true>(a, stream);
}

}  // namespace

bool chunked_supports(const FwdArgs& a) {
    if (a.dtype != 1 || (a.dk != 64 && a.dk != 128) || a.dv % DVT != 0 || a.dv < DVT) return false;
    // 16-byte direct copies of k, alpha, omega and v rows, 16-byte loads of k
    // rows (isotropic), 8-byte stores of four output columns
    return aligned16(a.q) && aligned16(a.k) && aligned16(a.v) && aligned16(a.alpha) && aligned16(a.omega) &&
           (reinterpret_cast<uintptr_t>(a.o) & 7u) == 0;
}

hipError_t launch_chunked_segments(const FwdArgs& a, int seg, int nseg, const float* mob, void* ophi, float* sseg,
                                   hipStream_t stream) {
    if (!chunked_supports(a) || a.variant != 0 || a.gates || a.cu_seqlens || seg <= 0 || seg % L != 0 || nseg < 1)
        return hipErrorNotSupported;
    bf16_t* op = static_cast<bf16_t*>(ophi);
    return a.dk == 128 ? launch_segments_t<128>(a, seg, nseg, mob, op, sseg, stream)
                       : launch_segments_t<64>(a, seg, nseg, mob, op, sseg, stream);
}

hipError_t launch_chunked(const FwdArgs& a, hipStream_t stream) {
    if (!chunked_supports(a)) return hipErrorNotSupported;
    if (a.variant == 3 && a.chunk_width == dvt_of<1>()) return hipErrorNotSupported;  // groups are 64 columns
    if (a.T == 0) return launch_recurrent(a, stream);  // only copies the initial state
    // the plain isotropic variant runs in its own kernel (kdn_iso.hip); the
    // isotropic chain below serves the per-channel-decay form (variant 2)
    if (a.variant == 1) return launch_iso(a, narrow_pays(a), stream);
    if (a.gates) {
        // the gate step inside (alpha, omega, r as pre-activations)
        if (a.variant == 3) return hipErrorNotSupported;
        return a.dk == 128 ? launch_gated<128>(a, stream) : launch_gated<64>(a, stream);
    }
    // variant 3: diagonal with grouped observation noise (one group per tile)
    if (a.dk == 128) {
        if (a.variant == 3) return launch_t<128, 0, true>(a, stream);
        if (narrow_pays(a)) {
            if (a.variant == 2) return launch_t<128, 2, false, 1>(a, stream);
            return launch_t<128, 0, false, 1>(a, stream);
        }
        if (a.variant == 2) return launch_t<128, 2>(a, stream);
        return launch_t<128, 0>(a, stream);
    }
    if (a.variant == 3) return launch_t<64, 0, true>(a, stream);
    if (narrow_pays(a)) {
        if (a.variant == 2) return launch_t<64, 2, false, 1>(a, stream);
        return launch_t<64, 0, false, 1>(a, stream);
    }
    if (a.variant == 2) return launch_t<64, 2>(a, stream);
    return launch_t<64, 0>(a, stream);
}

}  // namespace kdn
