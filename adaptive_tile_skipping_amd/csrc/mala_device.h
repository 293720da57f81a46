// Device-side helpers shared by the libmala kernels (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mala {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulate.
// Lane layouts (wave64): A[i][k] at lane i + 32*(k/8), element k%8;
// B[k][j] at lane j + 32*(k/8), element k%8;
// C[i][j] at lane j + 32*((i/4)%2), register (i/8)*4 + i%4.
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Same shape and layouts with fp16 operands.
__device__ __forceinline__ f32x16 mfma32x32x16_f16(const f16x8& a, const f16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x32) * B(32x16).  A[i][k] at lane i + 16*(k/8), element k%8;
// B[k][j] at lane j + 16*(k/8); C[i][j] at lane j + 16*(i/4), register i%4.
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Hardware base-2 exponential / logarithm (v_exp_f32, v_log_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }
__device__ __forceinline__ _Float16 to_f16(float x) { return (_Float16)x; }

// Two bf16 values (given as fp32 bit patterns) -> packed fp16.  Exact for
// magnitudes in fp16's normal range; beyond +-65504 the value saturates
// (round toward zero), below 2^-14 it becomes an fp16 subnormal.
__device__ __forceinline__ uint32_t pack2_f16_from_f32bits(uint32_t lo, uint32_t hi) {
    fp16x2 r = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(lo), __uint_as_float(hi));
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) { return __uint_as_float(b16 << 16); }

// The fp16 values in the low and high halves of a 32-bit word, as fp32.
__device__ __forceinline__ float f16_lo_to_float(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi_to_float(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Combine lane l with lane l^32.  v_permlane32_swap exchanges the upper half
// of one register with the lower half of another; applied to two copies of x
// it leaves {x[l % 32], x[l % 32 + 32]} in the two results of every lane, a
// VALU operation instead of an LDS-routed shuffle.  max and + are commutative,
// so the result is the same, bit for bit, as x op x[l ^ 32].
__device__ __forceinline__ float wave_max_pair(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sum_pair(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Position of key kk (0..15 within a 16-key group) in a transposed V tile
// (the forward's fp16 V copy): bits 2 and 3 swapped, so that the 8 consecutive positions a lane
// feeds to the P.V contraction are exactly the 8 keys its score registers hold.
__device__ __forceinline__ int vt_pos16(int kk) {
    return (kk & 3) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

// 16-byte global -> LDS copy that bypasses registers (gfx950
// global_load_lds_dwordx4).  Every lane supplies its own global address; the
// wave's 64 chunks land contiguously at `lds_wave_base` (wave-uniform), lane
// l at byte 16*l.
__device__ __forceinline__ void load16_to_lds(const void* gptr, void* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// LDS transposing read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element (i % 4) of the 8-byte chunks addressed by lanes
// 4k + i/4, k = 0..3.  So when lane j of a group addresses row r0 + j/4,
// columns c0 + 4 (j % 4) .. +3 of a 16-bit matrix, lane i receives rows
// r0..r0+3 of column c0 + i: four consecutive rows of one column.
// The result is returned as two dwords (elements 0-1, 2-3).
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* lds_elem) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) const uint16_t*)lds_elem));
    return __builtin_bit_cast(u32x2, x);
}

// Raw buffer resource over `nbytes` bytes at `base`, and the matching 16-byte
// global -> LDS copy at per-lane byte offset voffset.  The range check covers
// the per-lane offset: lanes whose 16 bytes lie past `nbytes` read zero, dword
// by dword.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}
__device__ __forceinline__ void buffer16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voffset, void* lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                            (int)voffset, 0, 0, 0);
}

// The same 16-byte copy issued from inline assembly, with the resource as four
// dwords (base, 48-bit; no stride; `nbytes` records; the flags above).  The
// range check covers voffset only: a nonzero wave-uniform soffset is added
// outside it, so use one only where every access stays inside the resource.  The
// compiler cannot see these as writes to LDS, so it adds none of its own waits
// for them before later LDS reads, which it otherwise does for any read it
// cannot prove disjoint from a copy in flight.  Every read of the destination
// must therefore follow an explicit s_waitcnt that covers the copy
// (wait_all_then_barrier).  The copy has no destination register, and the
// compiler's own partial vmcnt waits stay correct: operations it does not
// count only make an in-order counter wait longer.
__device__ __forceinline__ u32x4 raw_rsrc(const void* base, uint32_t nbytes) {
    const uint64_t b = (uint64_t)base;
    return u32x4{(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, nbytes, 0x00020000u};
}
__device__ __forceinline__ void buffer16_to_lds_asm(const u32x4& r, uint32_t voffset, uint32_t soffset,
                                                    void* lds_wave_base) {
    // the low 32 bits of a generic address into the LDS aperture are the LDS offset
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voffset), "s"(r), "s"(soffset), "{m0}"(m0)
                 : "memory");
}

// 16-byte global -> LDS copy (lane l's 16 bytes land at lds_wave_base + 16 l)
// from a 64-bit address, issued from inline assembly like buffer16_to_lds_asm:
// the compiler does not insert a wait for it before later LDS reads, so the
// caller waits (wait_vmcnt) for exactly the copies it needs.
__device__ __forceinline__ void global16_to_lds_asm(const void* gptr, void* lds_wave_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(m0) : "memory");
}

// Exchange point for data passed between the lanes of one wave through LDS:
// __builtin_amdgcn_wave_barrier() alone does not stop the compiler from moving
// memory accesses across it (it may hoist a lane's LDS read above the LDS write
// of another lane that it cannot see depends on it).  The memory clobber does;
// the LDS then executes the wave's accesses in issue order, and the wait makes
// this wave's earlier LDS operations complete first.
__device__ __forceinline__ void wave_lds_exchange() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

// Wait for every outstanding memory operation of this wave (including the
// global -> LDS copies above), then a workgroup barrier.
__device__ __forceinline__ void wait_all_then_barrier() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

// Wait until at most N vector-memory operations of this wave (loads, stores,
// global -> LDS copies; they retire in issue order) are outstanding.
// gfx9 s_waitcnt encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14].
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Maps a linear workgroup id onto a work-unit id so that `chunk` consecutive
// units run on the same XCD (workgroups are dealt round-robin to the 8 XCDs)
// while each XCD still receives units in increasing order.  Returns an id in
// [0, 8*chunk*ceil(n/(8*chunk))); ids >= n are padding and exit.
__device__ __forceinline__ int xcd_unit(int bid, int chunk) {
    const int xcd = bid & 7, slot = bid >> 3;
    return ((slot / chunk) * 8 + xcd) * chunk + slot % chunk;
}

}  // namespace mala
