// Vector loads and stores of the gfx950 kernels with explicit cache
// policies.
//
// Write-through stores.  A plain or non-temporal store leaves its line dirty
// in the L2 of the XCD that wrote it.  The line reaches HBM when L2 evicts
// it or, at the latest, when the release at the kernel's end writes every
// L2 back, and the next kernel on the stream waits for that write-back.  A
// store with system scope (sc0 sc1) goes through L2 to memory as it issues,
// so a kernel whose row stores all take that form leaves little to write
// back at its end.  The rows written here are read by later kernels only,
// which see them either way.
//
// The stores are inline assembly: no compiler builtin gives a plain store a
// cache scope.  The compiler does not see them as memory instructions, so
// the "memory" clobber keeps every other memory access on its side of the
// store, and the 16-byte form ends with one wait state (s_nop 0) because a
// VALU write to the data registers of a vector store wider than 8 bytes may
// not follow that store directly (a hazard the compiler checks only for the
// stores it emits itself).  Their completion counts in vmcnt like any other
// vector memory access; since the compiler does not count them, its own
// vmcnt waits can only wait longer than they would otherwise.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_ep {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 load16_nt(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ u32x2 load8_nt(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
}

__device__ __forceinline__ void store16_wt(void *p, u32x4 v)
{
    asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1\n\ts_nop 0" ::"v"(p), "v"(v) : "memory");
}

__device__ __forceinline__ void store8_wt(void *p, u32x2 v)
{
    asm volatile("global_store_dwordx2 %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
}

} // namespace moe_ep
