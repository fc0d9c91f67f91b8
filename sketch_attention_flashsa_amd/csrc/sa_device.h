// sa_device.h -- device helpers shared by the MFMA streaming kernels
// (sa_bf16_stream.hip, sa_fused_proj.hip, ...): MFMA and bf16 packing wrappers,
// counted memory waits, the direct-to-LDS load and the bare block barrier.
#pragma once

#include "sa_internal.h"

namespace sa {
namespace dev {

// Fast path of the online softmax while a lane's tile sum stays <= 2^16
// (relative to the running maximum); a larger sum takes the exact path.
constexpr float kLazyBound = 65536.0f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x2 pack2(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_convertvector(v, bf16x2);
}
__device__ __forceinline__ bf16x8 cat8(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
    bf16x4 lo = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    bf16x4 hi = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ float dot2sum(bf16x2 a, float acc) {
    const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(a, one, acc, false);
}
// k-slot j (0..7) of lane group g <-> row of the 32-row sub-tile
__device__ __forceinline__ int tok_of(int g, int j) { return (j < 4) ? 4 * g + j : 16 + 4 * g + (j - 4); }

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt[3:0],
// expcnt[6:4], lgkmcnt[11:8], vmcnt_hi[15:14]); the others are left at max.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// wait_vm<n * VMS> for a runtime n in [0, NMAX] (the counter operand is an immediate)
template <int NMAX, int VMS>
__device__ __forceinline__ void wait_after(int n) {
    if constexpr (NMAX == 0) {
        wait_vm<0>();
    } else {
        if (n >= NMAX) wait_vm<NMAX * VMS>();
        else wait_after<NMAX - 1, VMS>(n);
    }
}

// A wave-uniform pointer moved to scalar registers (readfirstlane of each
// half; the low half goes through uint32_t so it is zero-extended).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
    const uint64_t bb = (uint64_t)(uintptr_t)p;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(bb >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bb);
    return (T*)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
}

// The three direct-to-LDS loads below set M0 themselves and name it in their
// clobber lists, so that the compiler treats each asm statement as a writer
// of M0 and never keeps a value of its own there across one.  M0 is a
// register the compiler reserves, and clang warns about every reserved
// register in a clobber list; that warning is silenced for these statements
// only.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// One direct-to-LDS load of 16 bytes per lane: lane i's 16 bytes land at LDS
// address lds + 16*i (lds is wave-uniform; it goes through M0).  Written as
// asm so the compiler does not know that the ring is a DMA target and
// therefore never inserts its own (whole-ring) waits before LDS reads; the
// kernel's counted vmcnt waits are what orders the ring.  The asm has no
// output register, so nothing of it is left in flight in a register.  The
// source is a wave-uniform 64-bit base plus a per-lane 32-bit byte offset
// (lane i's 16 bytes come from base + voff).  The load is marked
// non-temporal: the streamed rows are read once, and the hint keeps them from
// displacing other lines in the caches (~2 % faster on the 100K-row workload).
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint32_t lds) {
    // uniform: pin it to SGPRs.  readfirstlane returns int: each half goes
    // through uint32_t so that the low half is zero-extended, not sign-extended.
    const uint64_t bb = (uint64_t)(uintptr_t)base;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(bb >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bb);
    const uint64_t ub = ((uint64_t)hi << 32) | (uint64_t)lo;
    base = (const void*)(uintptr_t)ub;
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1 nt"
        :
        : "v"(voff), "s"(base), "s"(lds)
        : "memory", "m0");
}

// Direct-to-LDS load as dma16s, without the non-temporal hint: for rows that
// several blocks read in turn, which should stay in the caches.
__device__ __forceinline__ void dma16c(const void* base, uint32_t voff, uint32_t lds) {
    const uint64_t bb = (uint64_t)(uintptr_t)base;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(bb >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bb);
    const uint64_t ub = ((uint64_t)hi << 32) | (uint64_t)lo;
    base = (const void*)(uintptr_t)ub;
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(base), "s"(lds)
        : "memory", "m0");
}

// Direct-to-LDS load of 4 bytes per lane (lane i's dword lands at lds + 4*i),
// otherwise as dma16c: for small per-row values that travel with a stage.
__device__ __forceinline__ void dma4c(const void* base, uint32_t voff, uint32_t lds) {
    const uint64_t bb = (uint64_t)(uintptr_t)base;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(bb >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bb);
    const uint64_t ub = ((uint64_t)hi << 32) | (uint64_t)lo;
    base = (const void*)(uintptr_t)ub;
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %0, %1"
        :
        : "v"(voff), "s"(base), "s"(lds)
        : "memory", "m0");
}

#pragma clang diagnostic pop

// 16-byte store that writes through to memory (system scope, non-temporal):
// for results written once at a kernel's end and read by the next kernel, so
// that they do not stay dirty in the caches and get written back in the
// middle of the following launch's reads.  The compiler's hazard tracking
// does not see into asm, and a VALU write of a store's data registers right
// after a store of more than 8 bytes is a hazard, so the asm ends with wait
// states before the compiler may reuse them.
__device__ __forceinline__ void store16_wt(f32x4* p, f32x4 v) {
    asm volatile(
        "global_store_dwordx4 %0, %1, off sc0 sc1 nt\n\t"
        "s_nop 7"
        :
        : "v"(p), "v"(v)
        : "memory");
}

// acc *= f in place, for an accumulator kept in AGPRs (the MFMA accumulator
// registers): each element goes through one VGPR and back, so the common
// path never copies the accumulator.
__device__ __forceinline__ void scale_in_place_acc(f32x4& acc, float f) {
    float t;
    asm volatile(
        "v_accvgpr_read_b32 %4, %0\n\t"
        "v_mul_f32 %4, %5, %4\n\t"
        "v_accvgpr_write_b32 %0, %4\n\t"
        "v_accvgpr_read_b32 %4, %1\n\t"
        "v_mul_f32 %4, %5, %4\n\t"
        "v_accvgpr_write_b32 %1, %4\n\t"
        "v_accvgpr_read_b32 %4, %2\n\t"
        "v_mul_f32 %4, %5, %4\n\t"
        "v_accvgpr_write_b32 %2, %4\n\t"
        "v_accvgpr_read_b32 %4, %3\n\t"
        "v_mul_f32 %4, %5, %4\n\t"
        "v_accvgpr_write_b32 %3, %4"
        : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "=&v"(t)
        : "v"(f));
}

// acc *= f in place.  A tied-operand ALU asm statement keeps the accumulator
// in the same registers on the (rare) rescale path, so the common path does
// not pay register copies to merge two versions of it.
__device__ __forceinline__ void scale_in_place(f32x4& acc, float f) {
    asm volatile(
        "v_mul_f32 %0, %4, %0\n\t"
        "v_mul_f32 %1, %4, %1\n\t"
        "v_mul_f32 %2, %4, %2\n\t"
        "v_mul_f32 %3, %4, %3"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
        : "v"(f));
}

// Bits j = 0..7 of a lane: validity of the rows of its PV k-slots.
__device__ __forceinline__ uint32_t lane_slots(uint32_t valid, int g) {
    return ((valid >> (4 * g)) & 0xFu) | (((valid >> (16 + 4 * g)) & 0xFu) << 4);
}

// Block barrier without the memory fence of __syncthreads (which would also
// wait for every DMA still in flight).  The empty asm statements only stop the
// compiler from moving memory accesses across the barrier; the counted waits
// before it make the stage's LDS contents complete.
__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}


}  // namespace dev
}  // namespace sa
