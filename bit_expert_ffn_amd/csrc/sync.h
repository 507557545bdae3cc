// Grid-wide barriers of the persistent kernels (one block per CU, every block resident): the
// single-launch layer and the fused routing kernel.  Internal header.
//
// The sync region is the first kSyncBytes of the workspace, in 32-bit words: arrival counters
// A, C and X and the error word, 64 bytes apart, the spin-limit word right after the error
// word; then kLsFlags copies of the "all arrived" flags of barriers A and C, 4 KB apart so that
// the pollers of different copies hit different memory channels.  A barrier: every block adds
// one to the barrier's counter (a relaxed device-scope atomic, issued after a full s_waitcnt so
// that this block's earlier device-scope stores are complete); the block that completes it
// raises every copy of the flag; each block polls its own copy.  Every wait is bounded.  At the
// exit every block adds one to counter X, and the last one resets the counters and flags: every
// call leaves them zero, whether or not its waits gave up.
#pragma once
#include "common.h"

namespace moe {

constexpr uint32_t kLsSpin = 1u << 21;    // default polls before a wait gives up (about 2 s)
constexpr int kLsSyncA = 0, kLsSyncC = 16, kLsSyncX = 32, kLsSyncErr = kSyncErrWord;
constexpr int kLsSyncSpin = kSyncSpinWord;
constexpr int kLsFlags = 16, kLsFlagBase = 64, kLsFlagStride = 1024;
constexpr int kLsFlagA = 0, kLsFlagC = 16;
static_assert((kLsFlagBase + (kLsFlags - 1) * kLsFlagStride + kLsFlagC + 1) * 4 <= kSyncBytes,
              "flags must fit in the sync region");

__device__ inline uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every earlier store of this block is complete, then thread 0 adds one to the counter; the
// block that brings it to G raises every copy of the barrier's flag.
__device__ inline void ls_arrive(uint32_t* sync, int ctr, int flag, uint32_t G) {
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  lds_barrier();
  if (threadIdx.x == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(sync + ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == G - 1)
      for (int i = 0; i < kLsFlags; ++i) st_dev(sync + kLsFlagBase + i * kLsFlagStride + flag, 1u);
  }
}

// Thread 0 polls this block's copy of the flag; the other wavefronts wait at an LDS-only
// barrier, keeping their own loads in flight.  false (for every thread) after `limit` polls.
__device__ inline bool ls_wait(uint32_t* sync, int flag, int* s_ok, uint32_t limit) {
  if (threadIdx.x == 0) {
    const uint32_t* f = sync + kLsFlagBase + (blockIdx.x % kLsFlags) * kLsFlagStride + flag;
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

// Exit, for a block that finished its work or gave up waiting: once this block's stores are
// complete, thread 0 arrives at counter X; the last block to arrive (every block has then
// stopped polling) resets the counters and flags for the next call.  The error word and the
// spin-limit word are left as they are.
__device__ inline void ls_exit(uint32_t* sync, uint32_t G) {
  if (threadIdx.x == 0) {
    __builtin_amdgcn_s_waitcnt(0);  // this block's flag stores are complete
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const uint32_t old =
        __hip_atomic_fetch_add(sync + kLsSyncX, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == G - 1) {
      st_dev(sync + kLsSyncA, 0u);
      st_dev(sync + kLsSyncC, 0u);
      for (int i = 0; i < kLsFlags; ++i) {
        st_dev(sync + kLsFlagBase + i * kLsFlagStride + kLsFlagA, 0u);
        st_dev(sync + kLsFlagBase + i * kLsFlagStride + kLsFlagC, 0u);
      }
      st_dev(sync + kLsSyncX, 0u);
    }
  }
}

}  // namespace moe
