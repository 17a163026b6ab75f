// Waits for direct global -> LDS tile loads (global_load_lds_dwordx4, gfx950).
//
// The kernels issue these loads as inline assembly with a wave-uniform
// scalar base and a 32-bit per-lane offset (each kernel's dma_lds16 /
// dma_asm16); lane l's 16 bytes land at the wave-uniform LDS address
// + 16*l.  The loads count against vmcnt, and the compiler does not see
// them as LDS writes, so every read of a stage follows an explicit
// s_waitcnt vmcnt(..) and an s_barrier (not __syncthreads, whose
// workgroup fence would drain every outstanding load).
#pragma once
#include "common.hpp"

namespace dmgqa {

// s_waitcnt vmcnt(n) with expcnt / lgkmcnt left unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

}  // namespace dmgqa
