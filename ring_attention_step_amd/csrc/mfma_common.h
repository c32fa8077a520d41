// Device helpers shared by the bf16 MFMA kernels (gfx950 / CDNA4): vector
// types, the LDS tile swizzle, bf16 packing, LDS-DMA issue and waits.
// Internal to libra.so.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ra {
namespace mfma {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

#define RA_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)((char*)(p)))
typedef __attribute__((address_space(3))) char lds_char;

// Chunk-position permutation of tile rows: 16-byte chunk c of tile row r is
// stored at chunk position c ^ swz(r).  gfx950's LDS serves 64 four-byte
// banks: swz is a bijection on 16 consecutive rows (so row-operand reads --
// 16 rows, one chunk each -- hit 16 distinct 16-byte bank groups) and gives 4
// consecutive rows disjoint 4-chunk spans (so ds_read_b64_tr_b16 reads -- 4
// rows x 4 chunks per 32 lanes -- are conflict free).
// D = 128: 16 chunks a row, swap the two 2-bit fields of r & 15.
// D = 64: 8 chunks a row (two rows per 64-bank line), bits 1..3 of r.
template <int D>
__device__ inline int swz(int r) {
    if (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
    return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// Eight fp32 accumulator values (base .. base + 7) -> one bf16 MFMA operand,
// round to nearest even (v_cvt_pk_bf16_f32).
__device__ inline bf16x8 pack_bf16x8(const f32x16& x, int base) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const f32x2 f = {x[base + e], x[base + e + 1]};
        const bf16x2 p = __builtin_convertvector(f, bf16x2);
        r[e] = p[0];
        r[e + 1] = p[1];
    }
    return r;
}

// s_waitcnt vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt left at "no wait").
__device__ inline void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(N): all but the N most recent vector-memory operations done.
template <int N>
__device__ inline void wait_vmem_leave() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// 16 bytes per lane HBM -> LDS (global_load_lds_dwordx4): lane l's bytes land at
// LDS byte address lds_base + 16 l.  Issued from inline assembly so that the
// compiler's wait-count pass does not treat the prefetch of the next tile as a
// hazard for reads of the current one; completion is awaited explicitly
// (wait_vmem_*) before the barrier that publishes a tile.
// The address is a wave-uniform base (SGPR pair) plus a 32-bit per-lane
// byte offset, so no per-lane 64-bit arithmetic is needed.
__device__ inline void lds_dma16(const void* base, uint32_t offset, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(offset), "s"(base), "s"(lds_base)
        : "memory", "m0");
}

// 4 bytes per lane HBM -> LDS (global_load_lds_dword); lane l's word lands at lds_base + 4 l.
__device__ inline void lds_dma4(const void* base, uint32_t offset, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %0, %1"
        :
        : "v"(offset), "s"(base), "s"(lds_base)
        : "memory", "m0");
}

// Work queues of persistent workgroups (see block_attn_mfma.hip): a tile
// space of n logical ids is cut into 8 queues, queue x holding the ids the
// fixed order places on XCD x; queue[0..7] are the queue heads, queue[8] the
// number of workgroups done claiming.
__device__ inline int xcd_queue_start(int x, int n) {
    const int q = n / 8, r = n % 8;
    return x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
}
// The next tile from this XCD's queue, else from another's; -1 when all are empty.
__device__ inline int claim_tile(uint32_t* queue, int n) {
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    for (int k = 0; k < 8; ++k) {
        const int x = static_cast<int>((xcc + k) & 7);
        const uint32_t size = static_cast<uint32_t>(xcd_queue_start(x + 1, n) - xcd_queue_start(x, n));
        const uint32_t i = __hip_atomic_fetch_add(queue + x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (i < size) return xcd_queue_start(x, n) + static_cast<int>(i);
    }
    return -1;
}
// Called once per workgroup (one lane) after its last, failed claim: the last
// workgroup of the grid zeroes the counters for the next launch.
__device__ inline void finish_claims(uint32_t* queue, uint32_t n_workgroups) {
    const uint32_t done = __hip_atomic_fetch_add(queue + 8, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == n_workgroups - 1) {
#pragma unroll
        for (int x = 0; x < 9; ++x) __hip_atomic_exchange(queue + x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace mfma
}  // namespace ra
