// cdna4.h -- small gfx950 (CDNA4) device helpers shared by the bf16 kernels:
// bf16 packing, the 32x32x16 and 16x16x32 bf16 MFMAs, buffer descriptors, direct-to-LDS
// buffer loads, the transposing LDS read and the wait + barrier hand-off.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {
namespace cdna4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const unsigned char lds_byte;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values -> two bf16 (round to nearest even), lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// D = A B + C on v_mfma_f32_32x32x16_bf16.  Lane l supplies row (A) or
// column (B) l % 32 and K elements 8 (l / 32) .. 8 (l / 32) + 7; the result
// lane l holds column l % 32, rows 8 (r / 4) + 4 (l / 32) + r % 4, r = 0..15.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Wait until at most N of this wave's vector-memory operations are in flight
// and its LDS operations are done, then meet the other waves at the barrier.
// The "memory" clobber keeps the compiler from moving LDS accesses across.
template <int N>
__device__ __forceinline__ void wait_then_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Buffer descriptor (gfx9 layout) over [base, base + range): 48-bit base,
// stride 0, byte range, and the raw 32-bit data-format word.  Loads past the
// range return zeros.  Every field is wave-uniform (SGPRs).
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t range)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xffffffffu));
    r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(range));
    r[3] = 0x00020000;
    return r;
}

// LDS byte address of a __shared__ array (or of an element of one), as the
// 32-bit value M0 and the LDS instructions take.
__device__ __forceinline__ uint32_t lds_addr(const unsigned char *shared)
{
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_byte *)shared));
}

// One wave-wide direct-to-LDS load: lane i's 16 bytes at byte offset voff of
// the buffer land at LDS byte address lds_dst + 16 i.  lds_dst is
// wave-uniform (lds_addr of the array plus uniform offsets, kept in SGPRs),
// so no per-lane address arithmetic is spent on it.  Issued as inline
// assembly so that the compiler does not track it: it would otherwise make
// every later LDS read wait for all loads in flight.  Completion is awaited
// explicitly (wait_then_barrier) before any wave reads the destination.  M0
// carries the LDS address; M0 is a register the compiler reserves for itself
// (a clobber declaration of it is not honoured), so the sequence saves M0 in
// a scratch SGPR and restores it after the load has issued (the load reads
// M0 at issue), leaving M0 as the compiler left it.  The instruction has no
// register result.
__device__ __forceinline__ void lds_dma16(i32x4 rsrc, uint32_t lds_dst, unsigned voff)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds_dst), "v"(voff), "s"(rsrc) : "memory");
}

// The same load with the non-temporal cache policy, for data that one call
// streams through exactly once (the decode's cache rows): the lines are not
// kept in the caches for reuse.
__device__ __forceinline__ void lds_dma16_stream(i32x4 rsrc, uint32_t lds_dst, unsigned voff)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds_dst), "v"(voff), "s"(rsrc) : "memory");
}

// D = A B + C on v_mfma_f32_16x16x32_bf16.  Lane l supplies row (A) or
// column (B) l % 16 and K elements 8 (l / 16) .. 8 (l / 16) + 7; the result
// lane l holds column l % 16, rows 4 (l / 16) + r, r = 0..3.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Transposing LDS read (gfx950): within each group of 16 lanes, lane j gets
// element (j & 3) of the 4 consecutive bf16 that lanes 4k + (j >> 2) address,
// for k = 0..3.  Packed two per dword, k = 0 in the low half of dword 0.
__device__ __forceinline__ u32x2 lds_read_tr4(const unsigned char *p)
{
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(lds_byte *)p);
    return __builtin_bit_cast(u32x2, v);
}

}  // namespace cdna4
}  // namespace mla
