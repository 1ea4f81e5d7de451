// Library-internal declarations of the kernel files: the host interface
// (rs_host.h) and the device-side arrival protocol of the step kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rs.h"
#include "rs_device.h"
#include "rs_host.h"

namespace rs {

// Per-sequence buffer counters, advanced inside the step kernels (sitech.ge
// ReplaySSM page, "How ReplaySSM works": append on a non-flush step; fold and
// clear on a flush; "Reducing state traffic and simplifying rollback": drafts
// held until verification). Every workgroup of a sequence first reads the
// sequence's counters; thread 0 then counts the workgroup in with a relaxed
// device-scope atomic whose operand depends on the values read, so it is
// issued only once the read has completed. Counting is two-level: workgroups
// arrive in groups of kArriveGroup on a counter of their own (one 128-byte
// line each, so that same-address atomics queue at most kArriveGroup deep;
// group sizes 4 to 32 time within 1%, the larger slightly ahead); the last
// of a group then arrives on the sequence's counter in rs_meta. The
// workgroup that arrives last there knows that all workgroups of its sequence
// have read the counters: it writes the advanced counters (or a sticky error
// bit, leaving them as they were, exactly as every workgroup skipped the
// sequence). Each last arriver clears the counter it closed for the next
// launch. The first-level atomic is issued after the state loads and its
// result is needed only at the end, so it costs the workgroup no wait.
enum class MetaOp { NonFlush = 0, Flush = 1, Append = 2 };

struct Arrival {
  uint32_t c;
  // wg: this workgroup's index among the nwg workgroups of its sequence;
  // ctr: the sequence's arrive_groups(nwg) first-level counters.
  __device__ __forceinline__ void arrive(uint32_t* ctr, int wg, long long nck, int len, int nd) {
    c = 0;
    if (threadIdx.x == 0) {
      uint32_t one = 1u;
      const int dep = static_cast<int>(nck) ^ len ^ nd;
      asm volatile("" : "+v"(one) : "v"(dep));   // the atomic waits for the counters read
      c = __hip_atomic_fetch_add(ctr + (wg / kArriveGroup) * kArriveStride, one, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // Called by every thread at the end; thread 0 of the last workgroup applies the rule.
  __device__ __forceinline__ void finish(rs_meta* m, uint32_t* ctr, int wg, int nwg, MetaOp op, int K,
                                         long long nck, int len, int nd) const {
    if (threadIdx.x != 0) return;
    const int g = wg / kArriveGroup;
    const int gsize = nwg - g * kArriveGroup < kArriveGroup ? nwg - g * kArriveGroup : kArriveGroup;
    if (c != static_cast<uint32_t>(gsize - 1)) return;
    __hip_atomic_store(ctr + g * kArriveStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int ng = arrive_groups(nwg);
    if (ng > 1) {
      const uint32_t c2 = __hip_atomic_fetch_add(&m->arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (c2 != static_cast<uint32_t>(ng - 1)) return;
      __hip_atomic_store(&m->arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    switch (op) {
      case MetaOp::NonFlush:
        if (nd != 0) m->err |= RS_ERR_PENDING;
        else if (len > kRing - 2) m->err |= RS_ERR_FULL;
        else m->len = len + 1;
        break;
      case MetaOp::Flush:
        if (nd != 0) m->err |= RS_ERR_PENDING;
        else if (len > kRing - 1) m->err |= RS_ERR_FULL;
        else {
          m->n_ckpt = nck + len + 1;
          m->len = 0;
        }
        break;
      case MetaOp::Append:
        if (nd != 0 || len + K > kRing) m->err |= RS_ERR_OVERFLOW;
        else m->nd = K;
        break;
    }
  }
};

}  // namespace rs
