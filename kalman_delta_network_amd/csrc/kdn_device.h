// kdn_device.h -- gfx950 device helpers shared by the chunked kernels: bf16
// conversions and packing, the matrix-core (MFMA) tile products and their
// operand orders, LDS tile swizzles, direct global -> LDS copies, barriers
// and waits, and the inverse of a chunk's two 16 x 16 lower-triangular
// diagonal blocks.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace kdn {
namespace dev {

typedef uint16_t bf16_t;
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
__device__ __forceinline__ float bf1(bf16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// float -> bf16, round to nearest even (hardware conversion on gfx950)
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    b2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}
// a * b + c as the three-operand form: the two-operand accumulate form would
// overwrite c, which for the chain's omega is a loop-carried input register
// that must keep its zero lower half (so the compiler would add a copy)
__device__ __forceinline__ float fma3(float a, float b, float c) {
    float r;
    asm("v_fma_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
// pack2 as one instruction the compiler cannot split again (it would convert
// each half on its own when the halves are stored separately)
__device__ __forceinline__ uint32_t pack2_opaque(float lo, float hi) {
    uint32_t r;
    asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
    return r;
}
__device__ __forceinline__ bf16_t to_bf(float x) {
    __bf16 b = (__bf16)x;
    return __builtin_bit_cast(bf16_t, b);
}
__device__ __forceinline__ s4 pack4(f4 x) {
    u2 u;
    u[0] = pack2(x[0], x[1]);
    u[1] = pack2(x[2], x[3]);
    return __builtin_bit_cast(s4, u);
}
__device__ __forceinline__ b8 pack8(f4 x, f4 y) {
    u4 u;
    u[0] = pack2(x[0], x[1]);
    u[1] = pack2(x[2], x[3]);
    u[2] = pack2(y[0], y[1]);
    u[3] = pack2(y[2], y[3]);
    return __builtin_bit_cast(b8, u);
}

// D = A B + C on one 16 x 16 tile.  16x16x32: lane l holds A[l%16][8(l/16)..+7],
// B[8(l/16)..+7][l%16] and C[4(l/16)..+3][l%16].  16x16x16: the same with
// 4 K values per lane.
__device__ __forceinline__ f4 mfma32(b8 a, b8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma16(s4 a, s4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// K-slot order of 16x16x32 operands.  A register operand built from two
// 16-row C tiles (rows 4g..4g+3 of each, lane group g) carries the K indices
// {32kk + 4g + j, 32kk + 16 + 4g + j}; LDS operands are stored with column i
// at position perm32(i) so that lane group g's 8 consecutive elements are
// the same K indices.
__device__ __forceinline__ int perm32(int i) {
    return (i & ~31) | ((i & 12) << 1) | ((i & 16) >> 2) | (i & 3);
}

// [rows][DK] bf16 tiles: 16-byte chunk c of row r sits at chunk c ^ r so that
// the 16 rows an MFMA operand read touches hit distinct banks.
template <int DK>
__device__ __forceinline__ int sw(int row, int col) {
    constexpr int NCH = DK / 8;
    return row * DK + ((((col >> 3) ^ row) & (NCH - 1)) << 3) + (col & 7);
}

// ---------------------------------------------------------------------------
// Cross-lane sums on VALU data moves, with no round trip through the LDS
// crossbar (a ds_bpermute chain costs its latency at every step, which a role
// run by one wave per SIMD cannot hide).  v_permlane32_swap exchanges lanes
// 32..63 of its first operand with lanes 0..31 of its second;
// v_permlane16_swap exchanges the odd 16-lane rows of its first operand with
// the even rows of its second.  DPP moves data inside a 16-lane row.  All 64
// lanes must be active.
// ---------------------------------------------------------------------------
// lanes 0..31: a[i] + a[i + 32]; lanes 32..63: b[i - 32] + b[i]
__device__ __forceinline__ float halve32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// lanes with bit 4 clear: a[i] + a[i + 16]; set: b[i - 16] + b[i]
__device__ __forceinline__ float halve16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i of each 8-lane half row <- lane 7 - i
constexpr int kDppRor8 = 0x128;       // lane i of each row <- lane (i + 8) mod 16, i.e. i ^ 8
// sum over the aligned group of 8 lanes, in each of them
__device__ __forceinline__ float sum8(float x) {
    x += dpp_mov<kDppXor1>(x);
    x += dpp_mov<kDppXor2>(x);
    return x + dpp_mov<kDppHalfMirror>(x);
}
// sum over the 16-lane row, in each of its lanes
__device__ __forceinline__ float sum16(float x) {
    x = sum8(x);
    return x + dpp_mov<kDppRor8>(x);
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int N>
struct IntC {
    static constexpr int value = N;
};

// Register prefetch rules (for the kernels' loaders).  Loaders issue
// unconditional loads from clamped addresses and never touch the loaded
// registers: a use inside a loader would make the compiler wait for each load
// in turn, and a load skipped on some path (a chunk index out of range) would
// make it wait for the newest loads before using older ones.  Chunk indices
// are clamped into [0, nchunks) (the kernels are never launched with T = 0)
// and tokens past the end of the sequence read the last token; both are
// masked where the values are used.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Asynchronous copies and synchronisation.
//
// g2lds16: direct global -> LDS copy of 16 bytes per lane (lane l's bytes from
// base + off_l land at dst + 16 l; base and dst uniform across the wave, so
// the address is a scalar base plus a 32-bit lane offset).  It is issued from
// inline assembly so that the compiler does not track it: the compiler
// otherwise waits for every such copy before the next LDS read, which would
// serialise the prefetch.  Untracked copies only make the compiler's own
// counter waits stricter (memory counters drain in order), never weaker.  The
// issuing wave waits for its copies with vm_wait<N>() before the barrier that
// precedes their use.  (The sub-dword forms of this load place one dword per
// lane, so they are not used for bf16 data.)
//
// bar(): workgroup barrier that waits for this wave's LDS traffic only.
// Global loads in flight (prefetches) and global stores (outputs nobody in
// the workgroup reads) may stay outstanding across it.
__device__ __forceinline__ void g2lds16(const void* base, uint32_t off, void* dst) {
    // both are uniform by construction; readfirstlane states it to the
    // compiler (its divergence analysis does not always see it), and costs
    // nothing for a value already in scalar registers
    // (readfirstlane returns int: each half goes back through uint32_t so the
    // low half is not sign-extended into the high one)
    const uint32_t lds =
        uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>((lds_void_t*)dst))));
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(b)));
    const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(b >> 32)));
    const uint64_t bu = (uint64_t(hi) << 32) | uint64_t(lo);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(bu), "s"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void bar() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Make the compiler wait for the load that produced x here, before any copy
// is issued: a wait it placed later would also drain the untracked copies.
template <class T>
__device__ __forceinline__ void settle(const T& x) {
    asm volatile("" ::"v"(x));
}

// Inverses of the two 16x16 diagonal blocks of M (in Md, fp32) into Td as
// bf16.  Each block is split into 8x8 sub-blocks,
//     [[P, 0], [C, Q]]^-1 = [[P^-1, 0], [-Q^-1 C P^-1, Q^-1]],
// so the sequential part is an 8-step substitution that runs for all four
// sub-blocks of the chunk at once (lanes 0..31), and the corner blocks are
// two small fp32 matrix-core products.  Md: both blocks column-major
// [a][s][t]; Wi: scratch for the 8x8 inverses; Td: both inverses as bf16
// [a][t][s], whose block (0,1) of each diagonal block is zero and written
// once by the caller.  One wave.
__device__ __forceinline__ void block_inverse(const float* Md, float (*Wi)[2][64], bf16_t* Td, int lane) {
    if (lane < 32) {
        // lane = (block a, sub-block w, column s): x solves P x = e_s (w = 0)
        // or Q x = e_s (w = 1) by forward substitution over the columns
        const int a = lane >> 4, w = (lane >> 3) & 1, s = lane & 7, o = 8 * w;
        const float* Mb = &Md[a * 256 + o * 16 + o];  // sub-block entry (t, u) at Mb[16 u + t]
        f4 col[8][2];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            col[u][0] = *reinterpret_cast<const f4*>(&Mb[16 * u]);
            col[u][1] = *reinterpret_cast<const f4*>(&Mb[16 * u + 4]);
        }
        float x[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) x[t] = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            // the unit right-hand side enters as a select (an indexed store
            // of a one-hot vector would go through scratch memory)
            x[u] = (x[u] + (u == s ? 1.f : 0.f)) * __builtin_amdgcn_rcpf(col[u][u / 4][u % 4]);
#pragma unroll
            for (int t = u + 1; t < 8; ++t) x[t] = fmaf(-col[u][t / 4][t % 4], x[u], x[t]);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) Td[a * 256 + (o + t) * 16 + o + s] = to_bf(x[t]);
        *reinterpret_cast<f4*>(&Wi[a][w][8 * s]) = f4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f4*>(&Wi[a][w][8 * s + 4]) = f4{x[4], x[5], x[6], x[7]};
    }
    wave_lds_sync();
    // corner blocks -Q^-1 (C P^-1) of both diagonal blocks together, as two
    // products of block-diagonal 16x16 fp32 matrices on the matrix cores
    // (index 8 a + t of those matrices is index t of block a).  Lane (j, n)
    // supplies row or column n and k-slot j; the second product takes its k
    // slots permuted (k = 4 j + i in step i) so that its right operand is
    // exactly the lane's accumulator of the first.
    const int n = lane & 15, j = lane >> 4;
    const int an = n >> 3, tn = n & 7;
    f4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k = 4 * i + j, ak = k >> 3, tk = k & 7;
        const float cv = Md[an * 256 + 16 * tk + 8 + tn];  // C of block an, [tn][tk]
        const float pv = Wi[ak][0][8 * tn + tk];           // P^-1 of block ak, [tk][tn]
        y = __builtin_amdgcn_mfma_f32_16x16x4f32(an == ak ? cv : 0.f, an == ak ? pv : 0.f, y, 0, 0, 0);
    }
    // y[e] = (C P^-1)[4 j + e][n] (block-diagonal)
    f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k = 4 * j + i, ak = k >> 3, tk = k & 7;
        const float qv = Wi[ak][1][8 * tk + tn];  // Q^-1 of block ak, [tn][tk]
        z = __builtin_amdgcn_mfma_f32_16x16x4f32(an == ak ? qv : 0.f, y[i], z, 0, 0, 0);
    }
    // z[e] = (Q^-1 C P^-1)[4 j + e][n]: rows and column in the same block form
    // row 4 (j & 1) + e, column tn of block an's corner
    if ((j >> 1) == an) {
#pragma unroll
        for (int e = 0; e < 4; ++e) Td[an * 256 + (8 + 4 * (j & 1) + e) * 16 + tn] = to_bf(-z[e]);
    }
}

}  // namespace dev
}  // namespace kdn
