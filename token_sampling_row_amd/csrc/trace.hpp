// Per-wavefront phase stamps, compiled only into the tracing build of the
// library (TSR_TRACE=1, libtsr_trace.so); in the ordinary build every stamp is
// an empty statement. Lane 0 of each wavefront records the 100 MHz real-time
// counter (s_memrealtime, the same clock on every compute unit) in LDS at
// each phase, and copies its record to the handle's buffer with ordinary
// vector stores when the row is done (trace[(block * waves + wave) * 16 +
// slot]): a store in flight would otherwise hold up the next barrier, which
// waits for the wavefront's outstanding memory operations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef TSR_TRACE
#define TSR_TRACE 0
#endif

namespace tsr {

constexpr int kTraceSlots = 16;     // phase slots per wavefront
constexpr int kTraceBlocks = 4096;  // workgroups traced per launch (the first ones)
constexpr int kTraceWaves = 8;      // wavefronts per workgroup recorded

// Slots of the sampler kernels (a slot a row does not reach stays 0).
enum : int {
  kStEntry = 0,      // kernel entry
  kStIssued = 1,     // row loads issued
  kStPassA = 2,      // pass A over the wavefront's last chunk done
  kStStats = 3,      // row statistics combined across the workgroup
  kStCompact1 = 4,   // first candidate compaction done
  kStSketch = 5,     // top-k candidate bound found
  kStCompact2 = 6,   // second compaction done
  kStResolve = 7,    // kept set resolved and token drawn (fast path)
  kStGeneral = 8,    // register-resident general search done
  kStWalk = 9,       // inverse-CDF walk done
  kStEnd = 10,       // outputs written
  kStStatsDone = 11, // row statistics returned (max, status, bounds combined)
  kStCutStart = 12,  // filters derived, kept-set search starting
  kStMask = 13,      // compaction: chunk rows holding candidates found
  kStCompactEnd = 14,  // compaction: this wavefront's candidates staged
  kStHwId = 15,      // not a time: XCC id << 16 | the low 16 bits of HW_ID
};

#if TSR_TRACE
// The stamp record of the workgroup, in its LDS.
struct TraceLds {
  unsigned long long t[kTraceWaves][kTraceSlots];
  unsigned long long* buf;   // the launch's buffer (null: not traced)
};

__device__ __forceinline__ void trace_begin(TraceLds& T, unsigned long long* buf) {
  const int w = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0 && w < kTraceWaves) {
    T.buf = buf;
#pragma unroll
    for (int s = 0; s < kTraceSlots; ++s) T.t[w][s] = 0ull;
    const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_REG_HW_ID
    const unsigned xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // HW_REG_XCC_ID
    T.t[w][kStHwId] = ((unsigned long long)(xcc & 0xFFFFu) << 16) | (hw & 0xFFFFu);
  }
}
__device__ __forceinline__ void trace_stamp(TraceLds& T, int slot) {
  const int w = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0 && w < kTraceWaves) T.t[w][slot] = __builtin_amdgcn_s_memrealtime();
}
__device__ __forceinline__ void trace_flush(TraceLds& T) {
  const int w = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0 && w < kTraceWaves && T.buf && blockIdx.x < (unsigned)kTraceBlocks) {
    unsigned long long* o = T.buf + ((unsigned long long)blockIdx.x * kTraceWaves + w) * kTraceSlots;
#pragma unroll
    for (int s = 0; s < kTraceSlots; ++s) o[s] = T.t[w][s];
  }
}
#endif

}  // namespace tsr
