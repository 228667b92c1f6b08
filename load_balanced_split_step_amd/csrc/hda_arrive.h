// Last-arriver counting across workgroups of one launch (device code).
//
// S workgroups that each store a partial result arrive at a shared 64-bit
// counter word; the one that arrives S-th combines the partials.  The word
// holds a fixed signature SIG in its high 32 bits and the arrivals of the
// current launch in its low 32; between launches it rests at (SIG, 0).  An
// arrival adds one (a single atomic, no retries: the workgroups of one
// output often arrive together, and an exchange loop paid a memory round
// trip per lost race).  A word not at rest -- memory no launch has used
// this way, whatever it holds -- is recognised by its high half and counted
// by compare-and-swap instead: the first exchange writes (SIG, 1), so the
// memory needs no clearing.  The last arriver puts the word back to rest,
// which keeps replays of a captured launch correct.
//
// Ordering is the caller's: each arriving workgroup makes its partial
// visible at agent scope before it arrives (a release fence), and the last
// one acquires before reading the others' partials.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

template <uint32_t SIG>
__device__ inline bool hda_arrive_last(unsigned long long* cnt, int S) {
  const unsigned long long rest = (unsigned long long)SIG << 32;
  const unsigned long long old = atomicAdd(cnt, 1ull);
  if ((old >> 32) == SIG && (uint32_t)old < (uint32_t)S) return (uint32_t)old == (uint32_t)(S - 1);
  // Each failed exchange returns the word as another arrival left it (at
  // most S - 1 counted arrivals and S - 1 additions to the stale word), or
  // once a stale guess, so 2 S attempts always suffice.
  unsigned long long cur = old + 1;
  for (int it = 0; it < 2 * S; ++it) {
    const unsigned long long next =
        ((cur >> 32) == SIG && (uint32_t)cur < (uint32_t)S) ? cur + 1 : rest + 1;
    const unsigned long long seen = atomicCAS(cnt, cur, next);
    if (seen == cur) return (uint32_t)next == (uint32_t)S;
    cur = seen;
  }
  return false;
}

// The last arriver's reset of the word to rest.
template <uint32_t SIG>
__device__ inline void hda_counter_rest(unsigned long long* cnt) {
  atomicExch(cnt, (unsigned long long)SIG << 32);
}
