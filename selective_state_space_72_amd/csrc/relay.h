// Hand-off of a state between two blocks of one launch (the "relay" that splits a work
// unit in time, part 1 continuing from part 0's final state).  Workgroups are dispatched
// in index order, so a waiting block's predecessor always has a smaller index and already
// holds a slot; the wait is bounded all the same, and a wait that gives up is made visible:
// it is counted in a fault word next to the flags (the host reads it back, see
// mamba_scan_fwd_relay_faults) and the receiving block continues from a NaN state, so every
// output that depends on the missing state is NaN rather than silently wrong.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mambascan {

// Polls of a normal relay wait (each about 8k cycles of s_sleep: a few seconds in all).
constexpr uint32_t kRelayPolls = 1u << 20;
// Polls when the planner runs the relay's failure test (part 0 withholds its hand-off).
constexpr uint32_t kRelayTestPolls = 1u << 10;

// Bounded wait for a relay flag (one thread of the block).  Polls with relaxed
// device-scope loads (no cache invalidation per poll, which would disturb every other
// wave on the XCD) and long sleeps, then acquires once.  True once the flag is raised,
// false after max_polls polls.
__device__ __forceinline__ bool relay_wait(uint32_t *flag, uint32_t max_polls)
{
    bool seen = false;
    for (uint32_t i = 0; i < max_polls; ++i) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
            seen = true;
            break;
        }
        __builtin_amdgcn_s_sleep(127);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return seen;
}

// Publish the state every thread of the block has stored: release its stores at device
// scope, then one thread raises the flag.
__device__ __forceinline__ void relay_signal(uint32_t *flag)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_store(flag, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// The waiting side: thread 0 waits, the block joins it, and every thread acquires before
// reading the state.  Returns, to every thread, whether the state arrived; a give-up adds
// one to *fault (a vector atomic of one lane).
__device__ __forceinline__ bool relay_receive(uint32_t *flag, uint32_t *fault, uint32_t max_polls)
{
    int missed = 0;
    if (threadIdx.x == 0) {
        missed = relay_wait(flag, max_polls) ? 0 : 1;
        if (missed)
            __hip_atomic_fetch_add(fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    missed = __syncthreads_or(missed);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return missed == 0;
}

} // namespace mambascan
