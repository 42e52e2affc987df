// bsr_device.hpp -- device helpers shared by the gfx950 kernels: vector types, bf16 rounding,
// raw buffer resources, direct-to-LDS loads, wait counters, LDS chunk swizzles, the 8-XCD
// work-group order and the bf16 matrix-core instructions.
//
// Matrix-core layouts (wave64):
//   v_mfma_f32_32x32x16_bf16: lane l holds A[l%32][8*(l/32) + t] and B[8*(l/32) + t][l%32], t = 0..7;
//     result item v of lane l is D[8*(v/4) + 4*(l/32) + v%4][l%32].
//   v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16) + t] and B[8*(l/16) + t][l%16];
//     result item v of lane l is D[4*(l/16) + v][l%16].
// Only the pairing of A's and B's k positions matters for the sum, so both operands always take
// the same k for the same (lane group, item).
//
// ds_read_b64_tr_b16 (transposing LDS read): in each group of 16 lanes, lane s supplies the
// address of 4 consecutive 16-bit values; lane i = 4u + v receives, as item t, value v of lane
// 4t + u. Pointing lane s at T[k0 + s/4][n0 + 4*(s%4)] of a row-major T[k][n] tile hands lane i
// the values T[k0..k0+3][n0 + i]: a k-run for one n, the matrix-core operand layout of a tile
// that is stored n-contiguous.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace bsr {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kCUs = 256;   // compute units of one MI355X
constexpr int kXCDs = 8;    // accelerator complex dies; work-groups go to them round-robin

// Logical index of work-group `bid` such that each XCD's work-groups (bid = x, x + 8, ...) take
// one contiguous run of logical indices, in dispatch order.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
    const int xcd = bid % kXCDs, slot = bid / kXCDs;
    const int per = nwg / kXCDs, rem = nwg % kXCDs;
    return xcd * per + min(xcd, rem) + slot;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 quad(const f32x16 &v, int q) { return f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]}; }

__device__ __forceinline__ uint16_t to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ float from_bf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ void store4_bf16(uint16_t *dst, float a, float b, float c, float d) {
    const uint32_t lo = (uint32_t)to_bf16(a) | ((uint32_t)to_bf16(b) << 16);
    const uint32_t hi = (uint32_t)to_bf16(c) | ((uint32_t)to_bf16(d) << 16);
    *reinterpret_cast<uint2 *>(dst) = make_uint2(lo, hi);
}

__device__ __forceinline__ f32x4 add_bias4(f32x4 v, const uint16_t *bias) {
    const uint2 bb = *reinterpret_cast<const uint2 *>(bias);
    v[0] += from_bf16(bb.x & 0xffff);
    v[1] += from_bf16(bb.x >> 16);
    v[2] += from_bf16(bb.y & 0xffff);
    v[3] += from_bf16(bb.y >> 16);
    return v;
}

// Buffer resources: a base address and a size in bytes. A buffer load whose offset lies past the
// size returns zeros and touches no memory, so loads can be issued unconditionally while rows past
// the end of a tile or absent blocks cost nothing.
constexpr int kBufferFlags = 0x00020000;   // raw 32-bit buffer, gfx9 layout

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufferFlags);
}

__device__ __forceinline__ bf16x8 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Byte offset in the work-group's LDS of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) void *)p;
}

// Direct-to-LDS load: lane i's 16 bytes at (voff, soff) of buffer r go to LDS byte address
// m0 + 16 i. Written as inline assembly so that the compiler, which cannot tell which LDS bytes
// such a load writes, does not wait for it before every LDS access; the kernels wait for these
// loads themselves (wait_vm) before the barrier that publishes a stage. The kernels that use it
// keep nothing else in M0.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t m0, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(m0), "v"(voff),
                 "s"(r), "s"(soff)
                 : "memory", "m0");
}

// Waits until at most n (wave-uniform, LO <= n <= HI) vector memory loads of this wave are in
// flight: a binary search over the immediate forms of s_waitcnt vmcnt.
template <int LO, int HI>
__device__ __forceinline__ void wait_vm(int n) {
    if constexpr (LO == HI) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LO) : "memory");
    } else {
        constexpr int MID = (LO + HI) / 2;
        if (n <= MID) wait_vm<LO, MID>(n);
        else wait_vm<MID + 1, HI>(n);
    }
}

// 16-byte chunk swizzles of staged tiles: chunk c of row r is stored at chunk c ^ swz(r), so that
// the 16-byte reads of a matrix-core operand (32 consecutive rows, one chunk each, per half-wave)
// spread over the LDS banks. Chosen by measurement on gfx950 (one CU, 16-byte reads of 32 rows x
// 2 chunks per wave, 8 waves): linear 1 KB reads 208 B/clk; rows of 8 chunks (128 bytes) with
// swz8 195 B/clk, unswizzled 36; rows of 4 chunks (64 bytes) with swz4 205 B/clk, with
// ((r >> 1) ^ (r >> 3)) & 3 133, unswizzled 72. The transposing 8-byte reads take 4 consecutive
// rows per group of 16 lanes and are conflict-free under any row-uniform chunk permutation.
__device__ __forceinline__ int swz8(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int swz4(int r) { return (r >> 2) & 3; }

}  // namespace dev
}  // namespace bsr
