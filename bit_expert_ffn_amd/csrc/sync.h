// Grid-wide barriers of the persistent kernels (one block per CU, every block resident): the
// single-launch layer and the fused routing kernel.  Internal header.
//
// The sync region is the first kSyncBytes of the workspace, in 32-bit words: the top-level
// arrival counters of barriers A, C and X and the error word, 64 bytes apart, the spin-limit
// word right after the error word; then kLsFlags copies of the "all arrived" flags of barriers
// A and C, 4 KB apart so that the pollers of different copies hit different memory channels;
// then the group counters, one 128-byte line each.  A barrier has two levels: every block adds
// one to the counter of its group (blocks b with the same b % 8, which the hardware places on
// one XCD), and the last arrival of each group adds one to the barrier's top-level counter; the
// block that completes that raises every copy of the flag, and each block polls its own copy.
// (Arrivals at one counter are serialised where the atomics execute: 256 of them on one word
// cost about 3 us, 32 on each of 8 words plus 8 on the top about a third of that.)  Every atomic
// is a relaxed device-scope one, issued after a full s_waitcnt so that the block's earlier
// device-scope stores are complete.  Every wait is bounded.  At the exit every block arrives
// at barrier X the same way, and the block that completes it resets every counter and flag:
// every call leaves them zero, whether or not its waits gave up.  (The single-launch kernel's
// per-XCD mode ends on its range counters instead: the arrival that completes the last range
// resets.)
#pragma once
#include "common.h"

namespace moe {

constexpr uint32_t kLsSpin = 1u << 21;    // default polls before a wait gives up (about 2 s)
constexpr int kLsSyncA = 0, kLsSyncC = 16, kLsSyncX = 32, kLsSyncErr = kSyncErrWord;
constexpr int kLsSyncSpin = kSyncSpinWord;
constexpr int kLsFlags = 16, kLsFlagBase = 64, kLsFlagStride = 1024;
constexpr int kLsFlagA = 0, kLsFlagC = 16;
constexpr int kLsGroups = 8;           // arrival groups: blocks with the same index mod 8
constexpr int kLsGroupBase = 15488;    // group counters: word kLsGroupBase + 32 (3 g + barrier)
static_assert((kLsFlagBase + (kLsFlags - 1) * kLsFlagStride + kLsFlagC + 1) < kLsGroupBase,
              "flags end before the group counters");
static_assert((kLsGroupBase + 32 * 3 * kLsGroups) * 4 <= kSyncBytes,
              "group counters must fit in the sync region");
// Group-local barrier C of the single-launch kernel's per-XCD mode (one counter and one flag per
// group) and its combine counters (one per range of output features), each on its own 128-byte
// line in the gaps between the first 8 flag copies.
constexpr int kLsXRanges = 32;  // combine counters: ranges of output features
__device__ inline uint32_t* ls_xc_ctr(uint32_t* sync, int g) { return sync + kLsFlagBase + g * kLsFlagStride + 256; }
__device__ inline uint32_t* ls_xc_flag(uint32_t* sync, int g) { return sync + kLsFlagBase + g * kLsFlagStride + 288; }
__device__ inline uint32_t* ls_xr_ctr(uint32_t* sync, int j) {
  return sync + kLsFlagBase + (j % kLsGroups) * kLsFlagStride + 512 + (j / kLsGroups) * 32;
}
// Per-XCD mode: ranges whose sum is complete (the arrival that completes the last one resets).
__device__ inline uint32_t* ls_xdone(uint32_t* sync) { return sync + kLsFlagBase + 640; }
static_assert(kLsXRanges <= 4 * kLsGroups, "combine counters: four lines per flag gap");
static_assert(kLsFlagBase + (kLsGroups - 1) * kLsFlagStride + 512 + 3 * 32 < kLsGroupBase,
              "per-XCD words end before the group counters");

__device__ inline uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The group counter of barrier `bar` (0: A, 1: C, 2: X) for group g.
__device__ inline uint32_t* ls_group_ctr(uint32_t* sync, int bar, int g) {
  return sync + kLsGroupBase + 32 * (3 * g + bar);
}

// Thread 0 only: this block's arrival at barrier `bar` (top-level counter word `top`) of a grid
// of G blocks; true for the one block whose arrival completes it.
__device__ inline bool ls_count(uint32_t* sync, int bar, int top, uint32_t G) {
  const uint32_t g = blockIdx.x % kLsGroups;
  const uint32_t gsize = G / kLsGroups + (g < G % kLsGroups ? 1u : 0u);
  const uint32_t old = __hip_atomic_fetch_add(ls_group_ctr(sync, bar, (int)g), 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
  if (old != gsize - 1) return false;
  const uint32_t ngroups = G < (uint32_t)kLsGroups ? G : (uint32_t)kLsGroups;
  return __hip_atomic_fetch_add(sync + top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
         ngroups - 1;
}

// Every earlier store of this block is complete, then thread 0 arrives; the block whose
// arrival completes the barrier raises every copy of its flag.
__device__ inline void ls_arrive(uint32_t* sync, int ctr, int flag, uint32_t G) {
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  lds_barrier();
  if (threadIdx.x == 0) {
    if (ls_count(sync, ctr == kLsSyncA ? 0 : 1, ctr, G))
      for (int i = 0; i < kLsFlags; ++i) st_dev(sync + kLsFlagBase + i * kLsFlagStride + flag, 1u);
  }
}

// Group barrier among the `gsize` blocks of group g: every earlier store of this block is
// complete, then thread 0 adds one to the group's counter; the last arrival raises its flag.
__device__ inline void ls_arrive_group(uint32_t* sync, int g, uint32_t gsize) {
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  lds_barrier();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(ls_xc_ctr(sync, g), 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    if (old == gsize - 1) st_dev(ls_xc_flag(sync, g), 1u);
  }
}

// Thread 0 polls the flag at `f`; the other wavefronts wait at an LDS-only barrier.  false (for
// every thread) after `limit` polls, with the error word set.
__device__ inline bool ls_wait_at(uint32_t* sync, const uint32_t* f, int* s_ok, uint32_t limit) {
  if (threadIdx.x == 0) {
    uint32_t spins = 0;
    int ok = 1;
    while (ld_dev(f) == 0) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > limit) {
        ok = 0;
        __hip_atomic_fetch_or(sync + kLsSyncErr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    *s_ok = ok;
  }
  lds_barrier();
  const bool ok = *s_ok != 0;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return ok;
}

// Thread 0 polls this block's copy of the flag; the other wavefronts wait at an LDS-only
// barrier, keeping their own loads in flight.  false (for every thread) after `limit` polls.
__device__ inline bool ls_wait(uint32_t* sync, int flag, int* s_ok, uint32_t limit) {
  return ls_wait_at(sync, sync + kLsFlagBase + (blockIdx.x % kLsFlags) * kLsFlagStride + flag, s_ok,
                    limit);
}

// Resets every counter and flag for the next call; called by one thread, once every block has
// stopped polling and every flag store is complete.  The error word and the spin-limit word are
// left as they are.
__device__ inline void ls_reset(uint32_t* sync) {
  st_dev(sync + kLsSyncA, 0u);
  st_dev(sync + kLsSyncC, 0u);
  for (int g = 0; g < kLsGroups; ++g) {
    for (int bar = 0; bar < 3; ++bar) st_dev(ls_group_ctr(sync, bar, g), 0u);
    st_dev(ls_xc_ctr(sync, g), 0u);
    st_dev(ls_xc_flag(sync, g), 0u);
  }
  for (int j = 0; j < kLsXRanges; ++j) st_dev(ls_xr_ctr(sync, j), 0u);
  st_dev(ls_xdone(sync), 0u);
  for (int i = 0; i < kLsFlags; ++i) {
    st_dev(sync + kLsFlagBase + i * kLsFlagStride + kLsFlagA, 0u);
    st_dev(sync + kLsFlagBase + i * kLsFlagStride + kLsFlagC, 0u);
  }
  st_dev(sync + kLsSyncX, 0u);
}

// Exit, for a block that finished its work or gave up waiting: once this block's stores are
// complete, thread 0 arrives at barrier X; the block that completes it (every block has then
// stopped polling) resets every counter and flag for the next call.
__device__ inline void ls_exit(uint32_t* sync, uint32_t G) {
  if (threadIdx.x == 0) {
    __builtin_amdgcn_s_waitcnt(0);  // this block's flag stores are complete
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (ls_count(sync, 2, kLsSyncX, G)) ls_reset(sync);
  }
}

}  // namespace moe
