// Per-wavefront phase stamps, compiled only into the tracing build of the
// library (TSR_TRACE=1, libtsr_trace.so); in the ordinary build every stamp is
// an empty statement. Lane 0 of each wavefront writes the 100 MHz real-time
// counter (s_memrealtime, the same clock on every compute unit) to
// trace[(block * kWaves + wave) * kTraceSlots + slot] with an ordinary vector
// store. The buffer belongs to the handle (sampler_trace_read).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef TSR_TRACE
#define TSR_TRACE 0
#endif

namespace tsr {

constexpr int kTraceSlots = 16;     // phase slots per wavefront
constexpr int kTraceBlocks = 4096;  // workgroups traced per launch (the first ones)

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
__device__ __forceinline__ void trace_stamp(unsigned long long* buf, int slot) {
  if (buf && (threadIdx.x & 63) == 0 && blockIdx.x < (unsigned)kTraceBlocks) {
    const unsigned long long t = __builtin_amdgcn_s_memrealtime();
    buf[((unsigned long long)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64) * kTraceSlots +
        slot] = t;
  }
}
// Where the wavefront runs: the accelerator complex die (XCC_ID) and the
// wave / SIMD / compute unit / shader array / engine fields of HW_ID.
__device__ __forceinline__ void trace_hw_id(unsigned long long* buf) {
  if (buf && (threadIdx.x & 63) == 0 && blockIdx.x < (unsigned)kTraceBlocks) {
    const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_REG_HW_ID
    const unsigned xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // HW_REG_XCC_ID
    buf[((unsigned long long)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64) * kTraceSlots +
        kStHwId] = ((unsigned long long)(xcc & 0xFFFFu) << 16) | (hw & 0xFFFFu);
  }
}
#define TSR_STAMP_P(buf, slot) ::tsr::trace_stamp((buf), (slot))
#else
#define TSR_STAMP_P(buf, slot) ((void)0)
#endif

}  // namespace tsr
