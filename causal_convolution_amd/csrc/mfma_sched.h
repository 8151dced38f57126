// Instruction-scheduling helpers shared by the MFMA kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace wanvae {

// sched_group_barrier instruction classes
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// A scheduling group of n (<= 9) instructions of class MASK: the builtin takes
// constant counts, and n is a constant once the caller's loops are unrolled.
template <int MASK>
__device__ inline void sched_group(int n) {
    switch (n) {
        case 1: __builtin_amdgcn_sched_group_barrier(MASK, 1, 0); break;
        case 2: __builtin_amdgcn_sched_group_barrier(MASK, 2, 0); break;
        case 3: __builtin_amdgcn_sched_group_barrier(MASK, 3, 0); break;
        case 4: __builtin_amdgcn_sched_group_barrier(MASK, 4, 0); break;
        case 5: __builtin_amdgcn_sched_group_barrier(MASK, 5, 0); break;
        case 6: __builtin_amdgcn_sched_group_barrier(MASK, 6, 0); break;
        case 7: __builtin_amdgcn_sched_group_barrier(MASK, 7, 0); break;
        case 8: __builtin_amdgcn_sched_group_barrier(MASK, 8, 0); break;
        case 9: __builtin_amdgcn_sched_group_barrier(MASK, 9, 0); break;
        default: break;
    }
}

}  // namespace wanvae
