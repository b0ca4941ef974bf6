// kdn_recurrent.hip -- token-by-token KDN recurrence for gfx950.
//
// One workgroup owns one (batch, head) pair and keeps its whole d_k x d_v
// memory S in registers for the full sequence.  Wave w owns the 32 value
// columns [32w, 32w + 32) and runs the per-token steps of
// kdn_recurrent_core.h on them (method steps 2-5 of the "Kalman Delta
// Networks" summary page, and the isotropic forms of its closing sentence);
// every column reduction over the key dimension stays inside one wave, so
// waves never wait for each other inside the token loop.
//
// Packed variable-length batches: unit b * H + h runs sequence b, whose
// tokens are rows [cu[b], cu[b + 1]) of the [T, H] token grid.
//
// The decode step is this kernel with T = 1 and the state updated in place:
// a barrier after the initial state loads makes every wave read p before any
// wave writes it back.
#include "kdn_gates.h"
#include "kdn_internal.h"
#include "kdn_recurrent_core.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kdn {
namespace {

typedef uint16_t bf16_t;  // raw bfloat16 bits

// VAR: 0 diagonal, 1 isotropic, 2 isotropic with per-channel decay.
// GR (diagonal only): grouped observation noise, one r and one uncertainty
// state p per group of 64 value columns (waves 2g, 2g + 1 form group g).
// NT: the carried state is read and written with nontemporal hints (states
// too large for the device's last-level cache, see kStreamStateBytes).
template <int DK, int DV, int VAR, typename Tin, bool GR = false, bool NT = false>
__global__ void __launch_bounds__(DV * 2)
kdn_recurrent_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                     const Tin* __restrict__ v, const Tin* __restrict__ alpha,
                     const Tin* __restrict__ omega, const Tin* __restrict__ r,
                     const float* __restrict__ c0, float mu, int T, int H, const float* S0,
                     const float* p0, Tin* __restrict__ o, float* S_T, float* p_T,
                     const int* __restrict__ cu, const int* __restrict__ ord, int nseq, int gates) {
    constexpr bool ISO = VAR != 0;       // one uncertainty scalar per head
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
            const dev::f4* src = reinterpret_cast<const dev::f4*>(S0 + sbase + size_t(i) * DV + col);
            const dev::f4 s4 = NT ? __builtin_nontemporal_load(src) : *src;
            S[m][0] = s4[0]; S[m][1] = s4[1]; S[m][2] = s4[2]; S[m][3] = s4[3];
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

    const rec::RecIO<Tin> io{q, k, v, alpha, omega, r, o, mu, H, DV, h, tok0, col, NG, grp, gates != 0};
    rec::run_tokens<DK, VAR, Tin, GR>(io, S, p, pb, chan[wave], 0, len);

#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + 8 * m;
        dev::f4* dst = reinterpret_cast<dev::f4*>(S_T + sbase + size_t(i) * DV + col);
        const dev::f4 sv = {S[m][0], S[m][1], S[m][2], S[m][3]};
        if (NT) __builtin_nontemporal_store(sv, dst);
        else *dst = sv;
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

// Carried states larger than this are streamed with nontemporal hints.
// MI355X's 256 MB last-level (Infinity) cache keeps much of a state of about
// its size between decode steps: the hints cost 9% per step at 256 sequences
// x 16 heads x 128 x 128 (268 MB) and save 8-9% at 512 and 1024 sequences
// (537 MB, 1.07 GB).
constexpr double kStreamStateBytes = 384.0 * 1024 * 1024;

template <int DK, int DV, int VAR, typename Tin, bool GR = false, bool NT = false>
hipError_t launch_nt(const FwdArgs& a, hipStream_t stream) {
    const long units = long(a.B) * a.H;
    hipLaunchKernelGGL((kdn_recurrent_kernel<DK, DV, VAR, Tin, GR, NT>), dim3(unsigned(units)),
                       dim3(DV * 2), 0, stream, static_cast<const Tin*>(a.q),
                       static_cast<const Tin*>(a.k), static_cast<const Tin*>(a.v),
                       static_cast<const Tin*>(a.alpha), static_cast<const Tin*>(a.omega),
                       static_cast<const Tin*>(a.r), a.c0, a.mu, a.T, a.H, a.S0, a.p0,
                       static_cast<Tin*>(a.o), a.S_T, a.p_T, a.cu_seqlens, a.seq_order, a.B,
                       a.gates ? 1 : 0);
    return hipGetLastError();
}

template <int DK, int DV, int VAR, typename Tin, bool GR = false>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
    const long units = long(a.B) * a.H;
    if (units == 0) return hipSuccess;
    const bool nt = double(units) * DK * DV * sizeof(float) > kStreamStateBytes;
    return nt ? launch_nt<DK, DV, VAR, Tin, GR, true>(a, stream) : launch_nt<DK, DV, VAR, Tin, GR, false>(a, stream);
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
