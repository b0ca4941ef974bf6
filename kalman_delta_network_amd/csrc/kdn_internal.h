// kdn_internal.h -- launcher interface between the C ABI (kdn_api.cpp) and the
// gfx950 kernels.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace kdn {

// One forward call, after host validation.  Pointers are device pointers.
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* alpha;
    const void* omega;
    const void* r;
    const float* c0;
    float mu;
    int variant;  // 0 diagonal, 1 isotropic, 2 isotropic with per-channel decay
    int dtype;    // 0 f32, 1 bf16
    int B, T, H, dk, dv;
    const float* S0;
    const float* p0;
    void* o;
    float* S_T;
    float* p_T;
    // packed variable-length batch: NULL for a [B,T,H] batch; otherwise B
    // sequences, sequence b owning tokens [cu_seqlens[b], cu_seqlens[b + 1])
    // of a [T,H] token grid (device pointer, B + 1 entries)
    const int* cu_seqlens = nullptr;
    // packed batch only: the order in which sequences are scheduled (device
    // pointer, B entries, a permutation of 0..B-1) or NULL for 0..B-1
    const int* seq_order = nullptr;
    // chunked forward: value columns per workgroup (64 or 32), 0 = chosen by
    // occupancy
    int chunk_width = 0;
    // diagonal variant: alpha, omega and r hold the gate pre-activations;
    // the kernels apply sigmoid, softplus and r_min + softplus themselves
    bool gates = false;
};

// One backward call, after host validation.  Pointers are device pointers;
// gradients are fp32 in the layouts of the inputs they belong to.
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* alpha;
    const void* omega;
    const void* r;
    const float* c0;
    float mu;
    int variant;  // as FwdArgs
    int dtype;    // 0 f32, 1 bf16 (of the token inputs and dO)
    int B, T, H, dk, dv;
    const float* S0;
    const float* p0;
    const void* dO;     // [B,T,H,dv] dtype, may be NULL (zero)
    const float* dS_T;  // may be NULL (zero)
    const float* dp_T;  // may be NULL (zero)
    float* dq;
    float* dk_;
    float* dv_;
    float* dalpha;
    float* domega;
    float* dr;
    float* dS0;
    float* dp0;
    float* dc0;   // may be NULL
    float* work;  // the workspace: work_bytes bytes, at least backward_workspace_bytes_for()
    size_t work_bytes = 0;
    // set by the chunked backward: flag[unit] = 1 for the (batch, head) pairs
    // the recurrent memory adjoint must take (their decays leave the chunked
    // form's range); the recurrent memory kernel then skips every other pair
    const int* only_flagged = nullptr;
    // chunked path only: alpha, omega, r hold the gate pre-activations and q,
    // k are raw (the kernels form the gated layer's values themselves)
    bool gates = false;
    // the token path's pairs in rounds: this call takes pairs slot0 ..
    // slot0 + nslot - 1, each in workspace slot (pair - slot0); nslot = 0
    // takes every pair at once (slot = pair)
    int slot0 = 0;
    int nslot = 0;
};

// Bytes of device workspace with which every variant and dtype runs with all
// its pairs at once (0 for an empty call).
size_t backward_workspace_bytes(int B, int T, int H, int dk, int dv);
// The smallest workspace a backward call of this variant and dtype accepts:
// the chunked path's layout (ChunkWs) where the diagonal bf16 form can take
// it, else backward_workspace_bytes.
size_t backward_workspace_bytes_for(int variant, int dtype, int B, int T, int H, int dk, int dv);
// Workspace of one (batch, head) pair on the token path (its rounds take as
// many pairs as the workspace holds).
size_t token_pair_bytes(int T, int dk, int dv);

// The chunked backward's workspace (diagonal bf16 form), carved from the
// caller's by chunk_workspace(); every region starts on 256 bytes, in this
// order.  The big per-token buffers hold one slab of tokens: the backward
// runs the slabs from the last, carrying dS and dp from one to the next.
struct ChunkWs {
    int* flag;          // [units] 1 where a chunk leaves the chunked form's range
    uint16_t* cks;      // [units][ntile][nchunks][dk / 4][64][4] bf16: diag(g_15) S at each chunk start
    float* ckp;         // [units][nchunks][dk]: p at each chunk start
    float* tsc;         // [units][T][8] per-token sums: u of tiles 0 and 1, d, dd, dr of the
                        // channel halves (2), 1 / |k| (gated), unused
    float* maps;        // [units][maxseg][dk][2]: the uncertainty adjoint's segment maps in one slab
    float* dpc;         // [2][units][dk]: dp carried between slabs (by slab parity)
    float* dsc;         // [units][dk][dv]: dS carried between slabs
    float* partial;     // [units][slab][ntile][4][dk]: per-token tile sums of one slab
    float* pbuf;        // [units][slab][dk]: p_{t-1} of one slab
    int slab;           // tokens per slab (a multiple of 32)
    int nslab;
    int maxseg;         // uncertainty segments per slab at most
    char* rest;         // everything after the flags (the token path's rounds reuse it)
    size_t rest_bytes;
};
// Layout in `bytes` bytes at `work`: the slab as long as fits (at least the
// minimum); false if even the minimum does not fit.
bool chunk_workspace(int B, int T, int H, int dk, int dv, void* work, size_t bytes, ChunkWs* out);
// Bytes of the chunked layout at its shortest slab.
size_t chunk_workspace_min_bytes(int B, int T, int H, int dk, int dv);
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream);
// The chunked path on its own (diagonal bf16 form; with a.gates the gated
// layer on raw q, k and pre-activations): the chunked adjoint for every pair
// in range, the token path with `fallback`'s arguments for the others, dc0.
// In two parts: main (checkpoints and the chunked adjoints; the flags of the
// pairs outside the chunked range are then at backward_chunk_flags) and
// fallback (the token path with `fallback`'s arguments for the flagged
// pairs, then dc0).
bool backward_chunked_eligible(const BwdArgs& a);
int* backward_chunk_flags(const BwdArgs& a);
hipError_t launch_backward_chunked_main(const BwdArgs& a, hipStream_t stream);
hipError_t launch_backward_chunked_fallback(const BwdArgs& a, const BwdArgs& fallback, hipStream_t stream);
// Backward of the gated layer: a.alpha, a.omega, a.r hold the gate
// pre-activations and d alpha, d omega, d r come out as their gradients.
// a.work holds backward_gated_workspace_bytes() bytes (the adjoint's
// workspace, then fp32 copies of the token inputs, the gated values and dO).
size_t backward_gated_workspace_bytes(int variant, int B, int T, int H, int dk, int dv);
// The smallest gated workspace for this variant and dtype: the adjoint's
// (backward_workspace_bytes_for) and the copies.
size_t backward_gated_workspace_bytes_for(int variant, int dtype, int B, int T, int H, int dk, int dv);
hipError_t launch_backward_gated(const BwdArgs& a, hipStream_t stream);

// kdn_backward_noalloc: the workspace is a static device array of this many
// bytes per device (kdn_noalloc.hip); noalloc_scratch() gives the current
// device's copy (its address resolved once per device, nothing allocated).
constexpr size_t kNoallocScratchBytes = size_t(256) << 20;
hipError_t noalloc_scratch(void** out);

// Token-by-token recurrence; one workgroup per (b, h) covering all d_v
// columns.  Also the decode step (T = 1, S_T == S0, p_T == p0 in place).
hipError_t launch_recurrent(const FwdArgs& a, hipStream_t stream);

// Chunkwise WY/UT forward on matrix cores.  Returns hipErrorNotSupported
// for shapes it does not handle (the caller then reports KDN_ERR_UNSUPPORTED).
bool chunked_supports(const FwdArgs& a);
hipError_t launch_chunked(const FwdArgs& a, hipStream_t stream);
// Compute units of the current device (cached per device; 256 if the query fails).
long device_cus();

// The diagonal forward of a long sequence cut into segments that run
// concurrently (kdn_split.hip).  split_segments: the number of segments used
// for these sizes (requested > 0: about that many; 0: chosen from the
// device's cus; 1: no split).  split_workspace_bytes: device workspace of a
// split with that many segments (0 when nseg < 2).  launch_split: the forward
// (nseg < 2: the plain chunked forward; the workspace is then unused).
int split_segments(int B, int T, int H, int dk, int dv, int requested, long cus);
size_t split_workspace_bytes(int B, int T, int H, int dk, int dv, int nseg);
hipError_t launch_split(const FwdArgs& a, int nseg, void* workspace, size_t workspace_bytes, hipStream_t stream);

// Segment mode of the diagonal chunked forward (kdn_split.hip drives it): the
// sequence cut into nseg segments of seg tokens (a multiple of 32) run
// concurrently; mob: [B*H][nseg][dk][4] Mobius products of the segments'
// uncertainty maps; ophi: [B*T][H][dk] bf16 outputs of the identity columns;
// sseg: [B*H][nseg][dk][dv + dk] segment end states.
hipError_t launch_chunked_segments(const FwdArgs& a, int seg, int nseg, const float* mob, void* ophi, float* sseg,
                                   hipStream_t stream);
// The chunked memory adjoint of the diagonal bf16 form (kdn_backward_chunk.hip)
// over chunks [c_lo, c_hi) of slab `slab`: one workgroup per (batch, head, 64
// value columns) whose flag is 0, reading the checkpoints
// launch_chunked_checkpoints wrote, writing the slab's per-token tile sums
// and p_{t-1}, the per-token sums, dv and (first slab) dS0.
hipError_t launch_backward_chunk(const BwdArgs& a, const ChunkWs& w, int slab, hipStream_t stream);
// The uncertainty adjoint of the same slab after launch_backward_chunk
// (per-channel waves); then, after the first slab, launch_backward_dr.
hipError_t launch_backward_unc_chunk(const BwdArgs& a, const ChunkWs& w, int slab, hipStream_t stream);
hipError_t launch_backward_dr(const BwdArgs& a, const ChunkWs& w, hipStream_t stream);
// Checkpoint sweep of the chunked backward (kdn_chunked.hip, diagonal bf16,
// d_v a multiple of 64): the memory in the midpoint frame, diag(g_15) S, in
// bf16 at every 32-token chunk start ([unit][tile][chunk][dk / 4][64][4] at
// cks) and p at every chunk start ([unit][chunk][dk] at ckp); ck_flag[unit] =
// 1 where a chunk leaves the chunked form's range (checkpoints stop there),
// else 0.
hipError_t launch_chunked_checkpoints(const FwdArgs& a, uint16_t* cks, float* ckp, int* ck_flag,
                                      hipStream_t stream);
// Chunkwise forward of the isotropic variant (variant 1) on Gram matrices of
// the raw keys (kdn_iso.hip); narrow = 32 value columns per workgroup, else 64.
// Same preconditions as launch_chunked, and T > 0.
hipError_t launch_iso(const FwdArgs& a, bool narrow, hipStream_t stream);

}  // namespace kdn
