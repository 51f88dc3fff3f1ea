// Hand-off of t between the workgroups of one launch, through the workspace's
// reserved region ("Execution paths", section "The GEMM formulation": the rank-r
// down-projection t = x V feeds the up-projection by U; where both run in one
// launch, the workgroups that compute t hand it to those that apply U).
//
// Producers (the first tgrid workgroups of the launch, dispatched before any
// waiter) write t with device-coherent stores and count themselves with one
// release increment of word kSyncArrive.  A waiter polls that word (bounded),
// acquires at agent scope, and counts itself as passed so that the counters can
// be zeroed for the next launch.  The passed counts are kept per group of
// waiters (the waiter's workgroup id modulo 8, which is also its XCD): one
// counter per group, each on its own 64-byte line, because increments of one
// word by every workgroup of a launch serialise at the memory side (~25 ns
// each, several microseconds for a few hundred workgroups finishing at once).
// The last waiter of a group counts the group in kSyncGroups; the last group
// zeroes everything, so every launch leaves the words at zero.
#pragma once

#include <hip/hip_runtime.h>

#include "aq_internal.h"

namespace aq {

struct HandoffWait {
  int wait_for;           // arrivals to wait for (tgrid)
  int spin;               // polls before the wait gives up
  int ngroups;            // groups with at least one waiter
  int gcount[kHandoffGroups];   // waiters per group
};

// Producer side, one thread, after every store of this workgroup completed.
__device__ __forceinline__ void handoff_arrive(unsigned *sync) {
  __hip_atomic_fetch_add(sync + kSyncArrive, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Waiter side, one thread of the workgroup; the caller follows with a
// workgroup barrier.  `first` is an arrival count read earlier (a poll issued
// ahead of the wait, to hide its latency).
__device__ __forceinline__ void handoff_wait_only(unsigned *sync, const HandoffWait &h, unsigned first) {
  bool seen = first >= (unsigned)h.wait_for;
  for (int it = 0; !seen && it < h.spin; ++it) {
    __builtin_amdgcn_s_sleep(2);
    seen = __hip_atomic_load(sync + kSyncArrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (unsigned)h.wait_for;
  }
  if (!seen) __hip_atomic_fetch_or(sync + kSyncFlag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // The producers released their t stores with their arrivals, and t is read
  // after this with plain loads, possibly on another XCD than the one that
  // wrote it: acquire at agent scope, so that no stale line of t is read.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Waiter side, one thread, any time after handoff_wait_only: counts this
// waiter as passed (`group` is blockIdx.x % 8); the last one zeroes the words.
__device__ __forceinline__ void handoff_pass(unsigned *sync, const HandoffWait &h, int group) {
  unsigned *gc = sync + kSyncGroup0 + kSyncGroupStride * group;
  if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 == (unsigned)h.gcount[group]) {
    __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__hip_atomic_fetch_add(sync + kSyncGroups, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 ==
        (unsigned)h.ngroups) {
      __hip_atomic_store(sync + kSyncArrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(sync + kSyncGroups, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Both, back to back.
__device__ __forceinline__ void handoff_wait(unsigned *sync, const HandoffWait &h, int group, unsigned first) {
  handoff_wait_only(sync, h, first);
  handoff_pass(sync, h, group);
}

__device__ __forceinline__ unsigned handoff_poll(const unsigned *sync) {
  return __hip_atomic_load(sync + kSyncArrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Host side: the waiters of a launch whose main workgroup j (blockIdx.x =
// tgrid + j, tgrid a multiple of 8) takes unit xcd_contiguous_tile(j, nunits);
// waits(u) tells whether unit u waits.  Fills the per-group counts.
template <class F>
inline void handoff_counts(int nunits, int tgrid, F waits, HandoffWait *h) {
  const int per = (nunits + kHandoffGroups - 1) / kHandoffGroups;
  h->ngroups = 0;
  for (int x = 0; x < kHandoffGroups; ++x) {
    int c = 0;
    for (int u = x * per; u < nunits && u < (x + 1) * per; ++u) c += waits(u) ? 1 : 0;
    h->gcount[x] = c;
    h->ngroups += c > 0 ? 1 : 0;
  }
  (void)tgrid;
  h->wait_for = tgrid + (debug_knob(AQ_DBG_HANDOFF_UNREACHABLE, 0) ? 1 : 0);
  h->spin = debug_knob(AQ_DBG_HANDOFF_SPIN, kHandoffSpin);
  if (h->spin < 1) h->spin = 1;
}

}  // namespace aq
