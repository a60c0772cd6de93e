// Direct buffer-to-LDS loads and the stage barrier of the LDS-pipelined
// fold kernels (forward, dx and dW_c).
//
// A stage of such a kernel is a set of wave-wide loads, each bringing 16
// bytes per lane from global memory straight into LDS (no registers, no LDS
// write instructions).  Stages are filled a few steps ahead into a ring of LDS
// buffers; before a wave reads a stage it waits until at most N of its own
// loads are still in flight and then joins the workgroup barrier, so every
// wave's part of the stage has landed.
//
// Range check: a raw buffer load returns zeros (and moves no data) when its
// per-lane offset plus the instruction offset reaches the descriptor's extent;
// the scalar offset is added to the address but is not part of that check.
// Every row or token offset that must fall past the extent (rows past M) is
// therefore carried in the per-lane offset, and the scalar offset only ever
// holds a position inside a row.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "ss1_device.h"

namespace ss1 {
namespace dev {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor over [base, base + bytes).
__device__ __forceinline__ i32x4 dma_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{static_cast<int>(a & 0xFFFFFFFFu), static_cast<int>((a >> 32) & 0xFFFFu), static_cast<int>(bytes),
                 kBufferWord3};
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// Per-lane offset that lies past every extent used here: such a load reads
// zeros (an absent plan source).
constexpr uint32_t kDmaAbsent = 0x7FFFFFFFu;

// One wave-wide load of 16 bytes per lane: lane l writes its 16 bytes at LDS
// byte address lds + 16*l.  Issued from inline asm: the instruction has no
// register result, and the compiler, which cannot tell these LDS writes apart
// from the operand reads of other stages, would otherwise wait for every one
// in flight before each LDS read.  The stage barriers order them instead; the
// memory clobber keeps LDS accesses on their side of the issue point.  M0 is
// listed as clobbered; nothing else in these kernels uses it (no LDS DMA
// builtins, no relative register indexing), and clang's note that a reserved
// register is not preserved across the statement is silenced here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(i32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voff),
                 "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Waits until at most N of this wave's buffer loads are in flight and its LDS
// reads are done, then joins the workgroup barrier.  A compiler fence here
// would wait for every direct-to-LDS load in flight (they count as LDS
// writes), which would drain the stage pipeline; the memory clobber keeps the
// compiler from moving LDS accesses across the barrier.
template <int N>
__device__ __forceinline__ void dma_stage_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// XOR key of LDS row p for rows of RB bytes stored as 16-byte pieces: piece
// i of row p sits at slot i ^ key(p).  The 16 rows that one quarter-wave
// reads at a given 16-byte column then land on 16 distinct bank groups.
template <int RB>
__device__ __forceinline__ int swz_key(int p) {
    return (p / (256 / RB)) % (RB / 16);
}

}  // namespace dev
}  // namespace ss1
