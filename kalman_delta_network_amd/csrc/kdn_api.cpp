// kdn_api.cpp -- the C ABI declared in include/kdn.h: host-side argument
// validation, algorithm dispatch and error reporting.  All device work is in
// the launchers of kdn_internal.h.
#include "kdn.h"
#include "kdn_internal.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return KDN_OK;
}

// Test hook: KDN_FAULT=launch makes every entry point report KDN_ERR_HIP
// after validation, without launching, so the error path can be exercised
// on a machine without a GPU.
bool fault_launch() {
    const char* f = std::getenv("KDN_FAULT");
    return f && std::strcmp(f, "launch") == 0;
}

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};

Span span(const void* p, size_t elems, size_t esize) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{lo, lo + elems * esize};
}

bool overlap(Span a, Span b) {
    if (a.lo == a.hi || b.lo == b.hi || a.lo == 0 || b.lo == 0) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

constexpr int64_t kMaxElems = int64_t(1) << 46;  // keeps every byte offset far from overflow

// both isotropic forms carry one uncertainty scalar per head
bool is_iso(int variant) { return variant == KDN_ISOTROPIC || variant == KDN_ISOTROPIC_CHANNEL; }

// entries of r per head-token (and of p per head and channel): one per group
// of 64 value columns for grouped observation noise, else one
size_t noise_groups(int variant, int dv) { return variant == KDN_DIAGONAL_GROUPED ? size_t(dv / 64) : 1; }

int validate_common(int variant, int dtype, float mu, int dk, int dv) {
    if (variant != KDN_DIAGONAL && variant != KDN_ISOTROPIC && variant != KDN_ISOTROPIC_CHANNEL &&
        variant != KDN_DIAGONAL_GROUPED)
        return fail(KDN_ERR_UNSUPPORTED, "unknown variant %d", variant);
    if (dtype != KDN_F32 && dtype != KDN_BF16) return fail(KDN_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    if (!std::isfinite(mu) || mu < 0.f) return fail(KDN_ERR_VALUE, "mu must be finite and >= 0 (got %g)", double(mu));
    if (dk < 0 || dv < 0) return fail(KDN_ERR_SHAPE, "negative head dimension (dk=%d, dv=%d)", dk, dv);
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128))
        return fail(KDN_ERR_UNSUPPORTED, "dk and dv must be 64 or 128 (got dk=%d, dv=%d)", dk, dv);
    return KDN_OK;
}

// Checks shared by the [B,T,H] forward and the packed forward: `units`
// (batch or sequence) x head pairs, `toks` token-head rows of the inputs,
// `cu` the packed offsets (NULL for [B,T,H]; `ncu` entries).
int validate_forward_core(const void* q, const void* k, const void* v, const void* alpha,
                          const void* omega, const void* r, const int* cu, int64_t ncu, const int* ord,
                          const float* c0, float mu, int variant, int dtype, int64_t units,
                          int64_t toks, int H, int dk, int dv, const float* S0, const float* p0,
                          void* o, float* S_T, float* p_T, int algo) {
    int st = validate_common(variant, dtype, mu, dk, dv);
    if (st != KDN_OK) return st;
    if (algo != KDN_ALGO_AUTO && algo != KDN_ALGO_RECURRENT && algo != KDN_ALGO_CHUNKED &&
        algo != KDN_ALGO_CHUNKED_WIDE && algo != KDN_ALGO_CHUNKED_NARROW)
        return fail(KDN_ERR_UNSUPPORTED, "unknown algorithm %d", algo);
    if (units == 0) return ok();  // nothing to read or write
    const bool iso = is_iso(variant);                      // one uncertainty scalar per head
    const size_t ng = noise_groups(variant, dv);           // r and p entries per head-token / head
    const bool chan = variant != KDN_ISOTROPIC;            // one decay per key channel
    if (toks > 0 && (!q || !k || !v || !alpha || !omega || !r || !o))
        return fail(KDN_ERR_NULL, "q, k, v, alpha, omega, r and o must be non-NULL");
    if (!S_T || !p_T) return fail(KDN_ERR_NULL, "S_T and p_T must be non-NULL");
    if (!c0 && !p0) return fail(KDN_ERR_NULL, "c0 may be NULL only when p0 is given");

    const size_t es = dtype == KDN_BF16 ? 2 : 4;
    const size_t nk = size_t(toks) * dk, nv = size_t(toks) * dv;
    const size_t na = chan ? nk : size_t(toks), nw = iso ? size_t(toks) : nk;
    const size_t ns = size_t(units) * dk * dv, np = iso ? size_t(units) : size_t(units) * ng * dk;
    const Span in[] = {span(q, nk, es),        span(k, nk, es),     span(v, nv, es),
                       span(alpha, na, es),    span(omega, nw, es), span(r, size_t(toks) * ng, es),
                       span(c0, size_t(H), 4), span(S0, ns, 4),     span(p0, np, 4),
                       span(cu, size_t(ncu), 4),   span(ord, size_t(ncu > 0 ? ncu - 1 : 0), 4)};
    const Span so = span(o, nv, es), sS = span(S_T, ns, 4), sp = span(p_T, np, 4);
    for (const Span& x : in) {
        if (overlap(so, x) || overlap(sp, x)) return fail(KDN_ERR_ALIAS, "an output overlaps an input");
        // S_T may be exactly S0 (continuation in place), nothing else
        if (overlap(sS, x) && !(x.lo == sS.lo && x.hi == sS.hi && S0 && x.lo == reinterpret_cast<uintptr_t>(S0)))
            return fail(KDN_ERR_ALIAS, "S_T overlaps an input other than S0 itself");
    }
    if (overlap(so, sS) || overlap(so, sp) || overlap(sS, sp))
        return fail(KDN_ERR_ALIAS, "outputs o, S_T, p_T overlap each other");
    return KDN_OK;
}

int validate_forward(const void* q, const void* k, const void* v, const void* alpha,
                     const void* omega, const void* r, const float* c0, float mu, int variant,
                     int dtype, int B, int T, int H, int dk, int dv, const float* S0,
                     const float* p0, void* o, float* S_T, float* p_T, int algo) {
    if (B < 0 || T < 0 || H < 0) return fail(KDN_ERR_SHAPE, "negative size (B=%d, T=%d, H=%d)", B, T, H);
    const int64_t units = int64_t(B) * H;
    const int64_t toks = units * T;
    if (units > INT32_MAX || toks > kMaxElems / 128)
        return fail(KDN_ERR_SHAPE, "problem too large (B=%d, T=%d, H=%d)", B, T, H);
    return validate_forward_core(q, k, v, alpha, omega, r, nullptr, 0, nullptr, c0, mu, variant, dtype, units,
                                 toks, H, dk, dv, S0, p0, o, S_T, p_T, algo);
}

int validate_forward_varlen(const void* q, const void* k, const void* v, const void* alpha,
                            const void* omega, const void* r, const int* cu_seqlens, const int* order,
                            const float* c0, float mu, int variant, int dtype, int N, int total,
                            int H, int dk, int dv, const float* S0, const float* p0, void* o,
                            float* S_T, float* p_T, int algo) {
    if (N < 0 || total < 0 || H < 0)
        return fail(KDN_ERR_SHAPE, "negative size (N=%d, total=%d, H=%d)", N, total, H);
    const int64_t units = int64_t(N) * H;
    const int64_t toks = int64_t(total) * H;
    if (units > INT32_MAX || toks > kMaxElems / 128)
        return fail(KDN_ERR_SHAPE, "problem too large (N=%d, total=%d, H=%d)", N, total, H);
    if (units > 0 && !cu_seqlens) return fail(KDN_ERR_NULL, "cu_seqlens must be non-NULL");
    return validate_forward_core(q, k, v, alpha, omega, r, cu_seqlens, int64_t(N) + 1, order, c0, mu, variant,
                                 dtype, units, toks, H, dk, dv, S0, p0, o, S_T, p_T, algo);
}

int validate_step(const void* q, const void* k, const void* v, const void* alpha, const void* omega,
                  const void* r, float mu, int variant, int dtype, int N, int H, int dk, int dv,
                  float* S, float* p, void* o) {
    int st = validate_common(variant, dtype, mu, dk, dv);
    if (st != KDN_OK) return st;
    if (N < 0 || H < 0) return fail(KDN_ERR_SHAPE, "negative size (N=%d, H=%d)", N, H);
    const int64_t units = int64_t(N) * H;
    if (units > INT32_MAX || units > kMaxElems / (128 * 128))
        return fail(KDN_ERR_SHAPE, "problem too large (N=%d, H=%d)", N, H);
    if (units == 0) return ok();
    if (!q || !k || !v || !alpha || !omega || !r || !o || !S || !p)
        return fail(KDN_ERR_NULL, "every pointer of kdn_step must be non-NULL");
    const bool iso = is_iso(variant), chan = variant != KDN_ISOTROPIC;
    const size_t ng = noise_groups(variant, dv);
    const size_t es = dtype == KDN_BF16 ? 2 : 4;
    const size_t nk = size_t(units) * dk, nv = size_t(units) * dv;
    const size_t na = chan ? nk : size_t(units), nw = iso ? size_t(units) : nk;
    const Span in[] = {span(q, nk, es), span(k, nk, es), span(v, nv, es),
                       span(alpha, na, es), span(omega, nw, es), span(r, size_t(units) * ng, es)};
    const Span so = span(o, nv, es), sS = span(S, size_t(units) * dk * dv, 4),
               sp = span(p, iso ? size_t(units) : nk * ng, 4);
    for (const Span& x : in)
        if (overlap(so, x) || overlap(sS, x) || overlap(sp, x))
            return fail(KDN_ERR_ALIAS, "the state or o overlaps a token input");
    if (overlap(so, sS) || overlap(so, sp) || overlap(sS, sp))
        return fail(KDN_ERR_ALIAS, "o, S and p overlap each other");
    return KDN_OK;
}

int validate_backward(const void* q, const void* k, const void* v, const void* alpha, const void* omega,
                      const void* r, const float* c0, float mu, int variant, int dtype, int B, int T,
                      int H, int dk, int dv, const float* S0, const float* p0, const void* dO,
                      const float* dS_T, const float* dp_T, float* dq, float* dk_out, float* dv_out,
                      float* dalpha, float* domega, float* dr, float* dS0, float* dp0, float* dc0,
                      void* work, size_t work_bytes, bool gated = false) {
    int st = validate_common(variant, dtype, mu, dk, dv);
    if (st != KDN_OK) return st;
    if (B < 0 || T < 0 || H < 0) return fail(KDN_ERR_SHAPE, "negative size (B=%d, T=%d, H=%d)", B, T, H);
    const int64_t units = int64_t(B) * H;
    const int64_t toks = units * T;
    // the memory kernel launches one workgroup per (batch, head, 64 value columns)
    if (units * (dv / 64) > INT32_MAX || toks > kMaxElems / 128)
        return fail(KDN_ERR_SHAPE, "problem too large (B=%d, T=%d, H=%d)", B, T, H);
    if (units == 0) return ok();
    const bool iso = is_iso(variant), chan = variant != KDN_ISOTROPIC;
    const size_t ng = noise_groups(variant, dv);
    if (toks > 0 && (!q || !k || !v || !alpha || !omega || !r))
        return fail(KDN_ERR_NULL, "q, k, v, alpha, omega and r must be non-NULL");
    if (toks > 0 && (!dq || !dk_out || !dv_out || !dalpha || !domega || !dr))
        return fail(KDN_ERR_NULL, "dq, dk, dv, dalpha, domega and dr must be non-NULL");
    if (!dS0 || !dp0) return fail(KDN_ERR_NULL, "dS0 and dp0 must be non-NULL");
    if (!c0 && !p0) return fail(KDN_ERR_NULL, "c0 may be NULL only when p0 is given");
    if (gated && variant == KDN_DIAGONAL_GROUPED)
        return fail(KDN_ERR_UNSUPPORTED, "no gate step with grouped observation noise (variant %d)", variant);
    const size_t need = gated ? kdn::backward_gated_workspace_bytes_for(variant, dtype, B, T, H, dk, dv)
                              : kdn::backward_workspace_bytes_for(variant, dtype, B, T, H, dk, dv);
    if (need > 0 && (!work || work_bytes < need))
        return fail(KDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, work_bytes);
    const auto mis16 = [](const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15u) != 0; };
    if (need > 0 && mis16(work)) return fail(KDN_ERR_WORKSPACE, "the workspace must be 16-byte aligned");
    const auto mis8 = [](const void* x) { return (reinterpret_cast<uintptr_t>(x) & 7u) != 0; };
    if (mis8(S0) || mis8(dS_T) || mis8(dS0) || mis8(dv_out))
        return fail(KDN_ERR_UNSUPPORTED, "S0, dS_T, dS0 and dv must be 8-byte aligned");

    const size_t es = dtype == KDN_BF16 ? 2 : 4;
    const size_t nk = size_t(toks) * dk, nv = size_t(toks) * dv;
    const size_t na = chan ? nk : size_t(toks), nw = iso ? size_t(toks) : nk;
    const size_t ns = size_t(units) * dk * dv, np = iso ? size_t(units) : size_t(units) * ng * dk;
    const Span in[] = {span(q, nk, es),     span(k, nk, es),        span(v, nv, es),
                       span(alpha, na, es), span(omega, nw, es),    span(r, size_t(toks) * ng, es),
                       span(c0, size_t(H), 4), span(S0, ns, 4),     span(p0, np, 4),
                       span(dO, nv, es),    span(dS_T, ns, 4),      span(dp_T, np, 4)};
    const Span out[] = {span(dq, nk, 4),     span(dk_out, nk, 4), span(dv_out, nv, 4),
                        span(dalpha, na, 4), span(domega, nw, 4), span(dr, size_t(toks) * ng, 4),
                        span(dS0, ns, 4),    span(dp0, np, 4),    span(dc0, size_t(H), 4),
                        span(work, need, 1)};
    for (size_t i = 0; i < sizeof(out) / sizeof(out[0]); ++i) {
        for (const Span& x : in)
            if (overlap(out[i], x)) return fail(KDN_ERR_ALIAS, "a gradient output or the workspace overlaps an input");
        for (size_t j = i + 1; j < sizeof(out) / sizeof(out[0]); ++j)
            if (overlap(out[i], out[j])) return fail(KDN_ERR_ALIAS, "gradient outputs or the workspace overlap each other");
    }
    return KDN_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    if (e == hipErrorNotSupported) return fail(KDN_ERR_UNSUPPORTED, "%s: shape not supported by this algorithm", what);
    return fail(KDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// launches a validated forward (a.cu_seqlens set for a packed batch)
int run_forward(kdn::FwdArgs a, hipStream_t s, int algo) {
    if (fault_launch()) return fail(KDN_ERR_HIP, "launch suppressed by KDN_FAULT=launch");
    if (algo == KDN_ALGO_CHUNKED || algo == KDN_ALGO_CHUNKED_WIDE || algo == KDN_ALGO_CHUNKED_NARROW) {
        if (!kdn::chunked_supports(a))
            return fail(KDN_ERR_UNSUPPORTED, "the chunked algorithm does not support this shape");
        a.chunk_width = algo == KDN_ALGO_CHUNKED_WIDE ? 64 : algo == KDN_ALGO_CHUNKED_NARROW ? 32 : 0;
        if (a.chunk_width == 32 && a.variant == KDN_DIAGONAL_GROUPED)
            return fail(KDN_ERR_UNSUPPORTED, "grouped observation noise needs 64-column workgroups");
        return hip_status(kdn::launch_chunked(a, s), "chunked forward");
    }
    if (algo == KDN_ALGO_AUTO && kdn::chunked_supports(a))
        return hip_status(kdn::launch_chunked(a, s), "chunked forward");
    return hip_status(kdn::launch_recurrent(a, s), "recurrent forward");
}

// Sizes of the split forward: the segments used and the workspace they need.
int split_nseg(int B, int T, int H, int dk, int dv, int segments) {
    return kdn::split_segments(B, T, H, dk, dv, segments, segments > 0 ? 0 : kdn::device_cus());
}

int validate_forward_split(const void* q, const void* k, const void* v, const void* alpha, const void* omega,
                           const void* r, const float* c0, float mu, int variant, int dtype, int B, int T, int H,
                           int dk, int dv, const float* S0, const float* p0, void* o, float* S_T, float* p_T,
                           int segments, void* work, size_t work_bytes) {
    int st = validate_forward(q, k, v, alpha, omega, r, c0, mu, variant, dtype, B, T, H, dk, dv, S0, p0, o, S_T,
                              p_T, KDN_ALGO_CHUNKED);
    if (st != KDN_OK) return st;
    if (variant != KDN_DIAGONAL || dtype != KDN_BF16)
        return fail(KDN_ERR_UNSUPPORTED, "the split forward takes the diagonal variant with bf16 inputs");
    if (segments < 0) return fail(KDN_ERR_VALUE, "segments must be >= 0 (got %d)", segments);
    if (int64_t(B) * H == 0 || T == 0) return KDN_OK;
    const int n = split_nseg(B, T, H, dk, dv, segments);
    const size_t need = kdn::split_workspace_bytes(B, T, H, dk, dv, n);
    if (need == 0) return KDN_OK;
    if (!work || work_bytes < need)
        return fail(KDN_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, work_bytes);
    if ((reinterpret_cast<uintptr_t>(work) & 15u) != 0)
        return fail(KDN_ERR_WORKSPACE, "the workspace must be 16-byte aligned");
    const size_t toks = size_t(B) * T * H, units = size_t(B) * H;
    const Span ws = span(work, need, 1);
    const Span other[] = {span(q, toks * dk, 2),      span(k, toks * dk, 2),     span(v, toks * dv, 2),
                          span(alpha, toks * dk, 2),  span(omega, toks * dk, 2), span(r, toks, 2),
                          span(c0, size_t(H), 4),     span(S0, units * dk * dv, 4), span(p0, units * dk, 4),
                          span(o, toks * dv, 2),      span(S_T, units * dk * dv, 4), span(p_T, units * dk, 4)};
    for (const Span& x : other)
        if (overlap(ws, x)) return fail(KDN_ERR_ALIAS, "the workspace overlaps an input or an output");
    return KDN_OK;
}

}  // namespace

extern "C" {

int kdn_forward_split_segments(int B, int T, int H, int dk, int dv, int segments) {
    if (B <= 0 || T <= 0 || H <= 0 || (dk != 64 && dk != 128) || (dv != 64 && dv != 128) || segments < 0) return 0;
    return split_nseg(B, T, H, dk, dv, segments);
}

size_t kdn_forward_split_workspace_size(int B, int T, int H, int dk, int dv, int segments) {
    if (B <= 0 || T <= 0 || H <= 0 || (dk != 64 && dk != 128) || (dv != 64 && dv != 128) || segments < 0) return 0;
    return kdn::split_workspace_bytes(B, T, H, dk, dv, split_nseg(B, T, H, dk, dv, segments));
}

int kdn_validate_forward_split(const void* q, const void* k, const void* v, const void* alpha, const void* omega,
                               const void* r, const float* c0, float mu, int variant, int dtype, int B, int T, int H,
                               int dk, int dv, const float* S0, const float* p0, void* o, float* S_T, float* p_T,
                               int segments, void* workspace, size_t workspace_bytes) {
    const int st = validate_forward_split(q, k, v, alpha, omega, r, c0, mu, variant, dtype, B, T, H, dk, dv, S0, p0,
                                          o, S_T, p_T, segments, workspace, workspace_bytes);
    return st == KDN_OK ? ok() : st;
}

int kdn_forward_split(const void* q, const void* k, const void* v, const void* alpha, const void* omega,
                      const void* r, const float* c0, float mu, int variant, int dtype, int B, int T, int H, int dk,
                      int dv, const float* S0, const float* p0, void* o, float* S_T, float* p_T, int segments,
                      void* workspace, size_t workspace_bytes, void* stream) {
    const int st = validate_forward_split(q, k, v, alpha, omega, r, c0, mu, variant, dtype, B, T, H, dk, dv, S0, p0,
                                          o, S_T, p_T, segments, workspace, workspace_bytes);
    if (st != KDN_OK) return st;
    if (int64_t(B) * H == 0) return ok();
    const kdn::FwdArgs a{q, k, v, alpha, omega, r, c0, mu, variant, dtype, B, T, H, dk, dv, S0, p0, o, S_T, p_T};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) return run_forward(a, s, KDN_ALGO_AUTO);
    if (fault_launch()) return fail(KDN_ERR_HIP, "launch suppressed by KDN_FAULT=launch");
    return hip_status(kdn::launch_split(a, split_nseg(B, T, H, dk, dv, segments), workspace, workspace_bytes, s),
                      "split forward");
}

int kdn_version(void) { return 600; }  // 0.6.0: the gated entry points normalise q and k

const char* kdn_status_string(int status) {
    switch (status) {
        case KDN_OK: return "ok";
        case KDN_ERR_NULL: return "a required pointer is NULL";
        case KDN_ERR_SHAPE: return "invalid size";
        case KDN_ERR_UNSUPPORTED: return "unsupported variant, dtype, head size or algorithm";
        case KDN_ERR_VALUE: return "invalid scalar argument";
        case KDN_ERR_HIP: return "HIP runtime error";
        case KDN_ERR_ALIAS: return "an output overlaps an input";
        case KDN_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        default: return "unknown status";
    }
}

const char* kdn_last_error(void) { return g_last_error; }

int kdn_validate_forward(const void* q, const void* k, const void* v, const void* alpha,
                         const void* omega, const void* r, const float* c0, float mu, int variant,
                         int dtype, int B, int T, int H, int dk, int dv, const float* S0,
                         const float* p0, void* o, float* S_T, float* p_T, int algo) {
    const int st = validate_forward(q, k, v, alpha, omega, r, c0, mu, variant, dtype, B, T, H, dk, dv,
                                    S0, p0, o, S_T, p_T, algo);
    return st == KDN_OK ? ok() : st;
}

int kdn_validate_step(const void* q, const void* k, const void* v, const void* alpha,
                      const void* omega, const void* r, float mu, int variant, int dtype, int N,
                      int H, int dk, int dv, float* S, float* p, void* o) {
    const int st = validate_step(q, k, v, alpha, omega, r, mu, variant, dtype, N, H, dk, dv, S, p, o);
    return st == KDN_OK ? ok() : st;
}

int kdn_forward_algo(const void* q, const void* k, const void* v, const void* alpha,
                     const void* omega, const void* r, const float* c0, float mu, int variant,
                     int dtype, int B, int T, int H, int dk, int dv, const float* S0,
                     const float* p0, void* o, float* S_T, float* p_T, void* stream, int algo) {
    const int st = validate_forward(q, k, v, alpha, omega, r, c0, mu, variant, dtype, B, T, H, dk,
                                    dv, S0, p0, o, S_T, p_T, algo);
    if (st != KDN_OK) return st;
    if (int64_t(B) * H == 0) return ok();
    const kdn::FwdArgs a{q, k, v, alpha, omega, r, c0, mu, variant, dtype, B, T, H, dk, dv,
                         S0, p0, o, S_T, p_T};
    return run_forward(a, static_cast<hipStream_t>(stream), algo);
}

int kdn_validate_forward_gated(const void* q, const void* k, const void* v, const void* z_alpha,
                               const void* z_omega, const void* z_r, const float* c0, float mu, int variant,
                               int dtype, int B, int T, int H, int dk, int dv, const float* S0,
                               const float* p0, void* o, float* S_T, float* p_T, int algo) {
    const int st = validate_forward(q, k, v, z_alpha, z_omega, z_r, c0, mu, variant, dtype, B, T, H, dk, dv,
                                    S0, p0, o, S_T, p_T, algo);
    if (st != KDN_OK) return st;
    if (variant == KDN_DIAGONAL_GROUPED)
        return fail(KDN_ERR_UNSUPPORTED, "no gate step with grouped observation noise (variant %d)", variant);
    return ok();
}

int kdn_forward_gated(const void* q, const void* k, const void* v, const void* z_alpha,
                      const void* z_omega, const void* z_r, const float* c0, float mu, int variant,
                      int dtype, int B, int T, int H, int dk, int dv, const float* S0,
                      const float* p0, void* o, float* S_T, float* p_T, void* stream, int algo) {
    const int st = kdn_validate_forward_gated(q, k, v, z_alpha, z_omega, z_r, c0, mu, variant, dtype, B, T, H,
                                              dk, dv, S0, p0, o, S_T, p_T, algo);
    if (st != KDN_OK) return st;
    if (int64_t(B) * H == 0) return ok();
    kdn::FwdArgs a{q, k, v, z_alpha, z_omega, z_r, c0, mu, variant, dtype, B, T, H, dk, dv,
                   S0, p0, o, S_T, p_T};
    a.gates = true;
    return run_forward(a, static_cast<hipStream_t>(stream), algo);
}

int kdn_validate_forward_varlen(const void* q, const void* k, const void* v, const void* alpha,
                                const void* omega, const void* r, const int* cu_seqlens,
                                const int* order, const float* c0, float mu, int variant, int dtype, int N, int total,
                                int H, int dk, int dv, const float* S0, const float* p0, void* o,
                                float* S_T, float* p_T, int algo) {
    const int st = validate_forward_varlen(q, k, v, alpha, omega, r, cu_seqlens, order, c0, mu, variant, dtype,
                                           N, total, H, dk, dv, S0, p0, o, S_T, p_T, algo);
    return st == KDN_OK ? ok() : st;
}

int kdn_forward_varlen(const void* q, const void* k, const void* v, const void* alpha,
                       const void* omega, const void* r, const int* cu_seqlens, const int* order,
                       const float* c0,
                       float mu, int variant, int dtype, int N, int total, int H, int dk, int dv,
                       const float* S0, const float* p0, void* o, float* S_T, float* p_T,
                       void* stream, int algo) {
    const int st = validate_forward_varlen(q, k, v, alpha, omega, r, cu_seqlens, order, c0, mu, variant, dtype,
                                           N, total, H, dk, dv, S0, p0, o, S_T, p_T, algo);
    if (st != KDN_OK) return st;
    if (int64_t(N) * H == 0) return ok();
    // N sequences over a [total, H] token grid: B = N, T = total, offsets on the device
    kdn::FwdArgs a{q, k, v, alpha, omega, r, c0, mu, variant, dtype, N, total, H, dk, dv,
                   S0, p0, o, S_T, p_T};
    a.cu_seqlens = cu_seqlens;
    a.seq_order = order;
    return run_forward(a, static_cast<hipStream_t>(stream), algo);
}

int kdn_forward_varlen_gated(const void* q, const void* k, const void* v, const void* z_alpha,
                             const void* z_omega, const void* z_r, const int* cu_seqlens, const int* order,
                             const float* c0, float mu, int variant, int dtype, int N, int total, int H, int dk,
                             int dv, const float* S0, const float* p0, void* o, float* S_T, float* p_T,
                             void* stream, int algo) {
    const int st = validate_forward_varlen(q, k, v, z_alpha, z_omega, z_r, cu_seqlens, order, c0, mu, variant,
                                           dtype, N, total, H, dk, dv, S0, p0, o, S_T, p_T, algo);
    if (st != KDN_OK) return st;
    if (variant == KDN_DIAGONAL_GROUPED)
        return fail(KDN_ERR_UNSUPPORTED, "no gate step with grouped observation noise (variant %d)", variant);
    if (int64_t(N) * H == 0) return ok();
    kdn::FwdArgs a{q, k, v, z_alpha, z_omega, z_r, c0, mu, variant, dtype, N, total, H, dk, dv,
                   S0, p0, o, S_T, p_T};
    a.cu_seqlens = cu_seqlens;
    a.seq_order = order;
    a.gates = true;
    return run_forward(a, static_cast<hipStream_t>(stream), algo);
}

int kdn_step_gated(const void* q, const void* k, const void* v, const void* z_alpha, const void* z_omega,
                   const void* z_r, float mu, int variant, int dtype, int N, int H, int dk, int dv,
                   float* S, float* p, void* o, void* stream) {
    const int st = validate_step(q, k, v, z_alpha, z_omega, z_r, mu, variant, dtype, N, H, dk, dv, S, p, o);
    if (st != KDN_OK) return st;
    if (variant == KDN_DIAGONAL_GROUPED)
        return fail(KDN_ERR_UNSUPPORTED, "no gate step with grouped observation noise (variant %d)", variant);
    if (int64_t(N) * H == 0) return ok();
    if (fault_launch()) return fail(KDN_ERR_HIP, "launch suppressed by KDN_FAULT=launch");
    kdn::FwdArgs a{q, k, v, z_alpha, z_omega, z_r, nullptr, mu, variant, dtype, N, 1, H, dk, dv,
                   S, p, o, S, p};
    a.gates = true;
    return hip_status(kdn::launch_recurrent(a, static_cast<hipStream_t>(stream)), "gated decode step");
}

int kdn_forward(const void* q, const void* k, const void* v, const void* alpha, const void* omega,
                const void* r, const float* c0, float mu, int variant, int dtype, int B, int T,
                int H, int dk, int dv, const float* S0, const float* p0, void* o, float* S_T,
                float* p_T, void* stream) {
    return kdn_forward_algo(q, k, v, alpha, omega, r, c0, mu, variant, dtype, B, T, H, dk, dv, S0,
                            p0, o, S_T, p_T, stream, KDN_ALGO_AUTO);
}

int kdn_step(const void* q, const void* k, const void* v, const void* alpha, const void* omega,
             const void* r, float mu, int variant, int dtype, int N, int H, int dk, int dv,
             float* S, float* p, void* o, void* stream) {
    const int st = validate_step(q, k, v, alpha, omega, r, mu, variant, dtype, N, H, dk, dv, S, p, o);
    if (st != KDN_OK) return st;
    if (int64_t(N) * H == 0) return ok();
    if (fault_launch()) return fail(KDN_ERR_HIP, "launch suppressed by KDN_FAULT=launch");
    // one token per sequence: the forward layouts with B = N, T = 1, state in place
    kdn::FwdArgs a{q, k, v, alpha, omega, r, nullptr, mu, variant, dtype, N, 1, H, dk, dv,
                   S, p, o, S, p};
    return hip_status(kdn::launch_recurrent(a, static_cast<hipStream_t>(stream)), "decode step");
}

size_t kdn_backward_workspace_size(int B, int T, int H, int dk, int dv) {
    if (B < 0 || T < 0 || H < 0 || dk < 0 || dv < 0) return 0;
    return kdn::backward_workspace_bytes(B, T, H, dk, dv);
}

size_t kdn_backward_workspace_size_for(int variant, int dtype, int B, int T, int H, int dk, int dv) {
    if (B < 0 || T < 0 || H < 0 || dk < 0 || dv < 0) return 0;
    return kdn::backward_workspace_bytes_for(variant, dtype, B, T, H, dk, dv);
}

int kdn_validate_backward(const void* q, const void* k, const void* v, const void* alpha,
                          const void* omega, const void* r, const float* c0, float mu, int variant,
                          int dtype, int B, int T, int H, int dk, int dv, const float* S0,
                          const float* p0, const void* dO, const float* dS_T, const float* dp_T,
                          float* dq, float* dk_out, float* dv_out, float* dalpha, float* domega,
                          float* dr, float* dS0, float* dp0, float* dc0, void* workspace,
                          size_t workspace_bytes) {
    const int st = validate_backward(q, k, v, alpha, omega, r, c0, mu, variant, dtype, B, T, H, dk, dv, S0, p0,
                                     dO, dS_T, dp_T, dq, dk_out, dv_out, dalpha, domega, dr, dS0, dp0, dc0,
                                     workspace, workspace_bytes);
    return st == KDN_OK ? ok() : st;
}

int kdn_backward(const void* q, const void* k, const void* v, const void* alpha, const void* omega,
                 const void* r, const float* c0, float mu, int variant, int dtype, int B, int T,
                 int H, int dk, int dv, const float* S0, const float* p0, const void* dO,
                 const float* dS_T, const float* dp_T, float* dq, float* dk_out, float* dv_out,
                 float* dalpha, float* domega, float* dr, float* dS0, float* dp0, float* dc0,
                 void* workspace, size_t workspace_bytes, void* stream) {
    const int st = validate_backward(q, k, v, alpha, omega, r, c0, mu, variant, dtype, B, T, H, dk, dv, S0, p0,
                                     dO, dS_T, dp_T, dq, dk_out, dv_out, dalpha, domega, dr, dS0, dp0, dc0,
                                     workspace, workspace_bytes);
    if (st != KDN_OK) return st;
    if (int64_t(B) * H == 0) return ok();
    if (fault_launch()) return fail(KDN_ERR_HIP, "launch suppressed by KDN_FAULT=launch");
    const kdn::BwdArgs a{q, k, v, alpha, omega, r, c0, mu, variant, dtype, B, T, H, dk, dv, S0, p0, dO, dS_T,
                         dp_T, dq, dk_out, dv_out, dalpha, domega, dr, dS0, dp0, dc0,
                         static_cast<float*>(workspace), workspace_bytes};
    return hip_status(kdn::launch_backward(a, static_cast<hipStream_t>(stream)), "backward");
}

int kdn_backward_noalloc(const void* q, const void* k, const void* v, const void* alpha, const void* omega,
                         const void* r, const float* c0, float mu, int variant, int dtype, int B, int T, int H,
                         int dk, int dv, const float* S0, const float* p0, const void* dO, const float* dS_T,
                         const float* dp_T, float* dq, float* dk_out, float* dv_out, float* dalpha, float* domega,
                         float* dr, float* dS0, float* dp0, float* dc0, void* stream) {
    // the checks of kdn_backward, with the static scratch standing for the
    // workspace: its size first (no device access), then its address
    int st = validate_common(variant, dtype, mu, dk, dv);
    if (st != KDN_OK) return st;
    if (B < 0 || T < 0 || H < 0) return fail(KDN_ERR_SHAPE, "negative size (B=%d, T=%d, H=%d)", B, T, H);
    const size_t need = kdn::backward_workspace_bytes_for(variant, dtype, B, T, H, dk, dv);
    if (need > kdn::kNoallocScratchBytes)
        return fail(KDN_ERR_WORKSPACE,
                    "kdn_backward_noalloc: these sizes need %zu bytes of workspace, more than the %zu-byte static "
                    "scratch (use kdn_backward with a workspace)", need, kdn::kNoallocScratchBytes);
    if (fault_launch()) return fail(KDN_ERR_HIP, "launch suppressed by KDN_FAULT=launch");
    void* scratch = nullptr;
    if (need > 0 && int64_t(B) * H > 0) {
        const hipError_t e = kdn::noalloc_scratch(&scratch);
        if (e != hipSuccess) return fail(KDN_ERR_HIP, "kdn_backward_noalloc: device scratch: %s", hipGetErrorString(e));
    }
    return kdn_backward(q, k, v, alpha, omega, r, c0, mu, variant, dtype, B, T, H, dk, dv, S0, p0, dO, dS_T, dp_T, dq,
                        dk_out, dv_out, dalpha, domega, dr, dS0, dp0, dc0, scratch, scratch ? need : 0, stream);
}

size_t kdn_backward_gated_workspace_size(int variant, int B, int T, int H, int dk, int dv) {
    if (B < 0 || T < 0 || H < 0 || dk < 0 || dv < 0 || variant < 0 || variant > 2) return 0;
    return kdn::backward_gated_workspace_bytes(variant, B, T, H, dk, dv);
}

size_t kdn_backward_gated_workspace_size_for(int variant, int dtype, int B, int T, int H, int dk, int dv) {
    if (B < 0 || T < 0 || H < 0 || dk < 0 || dv < 0 || variant < 0 || variant > 2) return 0;
    return kdn::backward_gated_workspace_bytes_for(variant, dtype, B, T, H, dk, dv);
}

int kdn_backward_gated(const void* q, const void* k, const void* v, const void* z_alpha, const void* z_omega,
                       const void* z_r, const float* c0, float mu, int variant, int dtype, int B, int T,
                       int H, int dk, int dv, const float* S0, const float* p0, const void* dO,
                       const float* dS_T, const float* dp_T, float* dq, float* dk_out, float* dv_out,
                       float* dz_alpha, float* dz_omega, float* dz_r, float* dS0, float* dp0, float* dc0,
                       void* workspace, size_t workspace_bytes, void* stream) {
    const int st = validate_backward(q, k, v, z_alpha, z_omega, z_r, c0, mu, variant, dtype, B, T, H, dk, dv, S0,
                                     p0, dO, dS_T, dp_T, dq, dk_out, dv_out, dz_alpha, dz_omega, dz_r, dS0, dp0,
                                     dc0, workspace, workspace_bytes, true);
    if (st != KDN_OK) return st;
    if (int64_t(B) * H == 0) return ok();
    if (fault_launch()) return fail(KDN_ERR_HIP, "launch suppressed by KDN_FAULT=launch");
    const kdn::BwdArgs a{q, k, v, z_alpha, z_omega, z_r, c0, mu, variant, dtype, B, T, H, dk, dv, S0, p0, dO, dS_T,
                         dp_T, dq, dk_out, dv_out, dz_alpha, dz_omega, dz_r, dS0, dp0, dc0,
                         static_cast<float*>(workspace), workspace_bytes};
    return hip_status(kdn::launch_backward_gated(a, static_cast<hipStream_t>(stream)), "gated backward");
}

}  // extern "C"
