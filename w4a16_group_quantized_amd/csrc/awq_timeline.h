// Per-wave timestamps for the timeline probe.  The library is built without
// AWQ_TIMELINE and everything here expands to nothing.  probes/timeline.hip
// defines AWQ_TIMELINE, compiles the same kernels with their stamps (the
// constant 100 MHz counter s_memrealtime, and s_memtime, the shader clock) and
// defines the array they go to: awq_timeline[field][slot], one slot per
// recording wave.
#pragma once

#ifdef AWQ_TIMELINE
constexpr int kTimelineSlots = 8192;
constexpr int kTimelineFields = 6;
extern __device__ unsigned long long awq_timeline[kTimelineFields][kTimelineSlots];

#define AWQ_TL_STAMP(name) const unsigned long long name = __builtin_amdgcn_s_memrealtime()
#define AWQ_TL_CLOCK(name) const unsigned long long name = __builtin_amdgcn_s_memtime()

__device__ __forceinline__ void awq_tl_record(int slot, unsigned long long f0, unsigned long long f1,
                                              unsigned long long f2, unsigned long long f3,
                                              unsigned long long f4, unsigned long long f5) {
    if (slot < 0 || slot >= kTimelineSlots) return;
    awq_timeline[0][slot] = f0;
    awq_timeline[1][slot] = f1;
    awq_timeline[2][slot] = f2;
    awq_timeline[3][slot] = f3;
    awq_timeline[4][slot] = f4;
    awq_timeline[5][slot] = f5;
}
#else
#define AWQ_TL_STAMP(name)
#define AWQ_TL_CLOCK(name)
#endif
