// Phase timestamps for the benchmark's traced build of the decode kernel
// (libpkv_trace.so). Included by pkv_decode.hip inside its own namespace; the
// normal build defines PKV_PHASE and PKV_PHASE_VALUE as empty statements.
#pragma once

// Phase timestamps (the benchmark's traced build, libpkv_trace.so, compiled
// with PKV_PHASE_TRACE): wave 0 of each workgroup records the 100 MHz
// realtime counter at the phase boundaries of the decode kernel into one row
// per linear workgroup id. Phases: 0 entry, 1 piece and context length known,
// 2 queries and block ids arrived, 3 first K/V tile in LDS, 4 tiles done,
// 5 partial stored, 6 stores acknowledged, 7 counted, 8 end; slot 9 is 1 if
// the workgroup merged, slot 10 counts its pieces. A workgroup that runs
// several pieces (stream-K ranges) keeps phases 1-7 of its first piece and
// the end of its last. The normal build compiles all of this away.
#ifdef PKV_PHASE_TRACE
constexpr int kTraceRows = 1 << 16, kTraceCols = 11;
__device__ unsigned long long g_phase_trace[kTraceRows][kTraceCols];
__device__ __forceinline__ unsigned long long phase_clock() {
  unsigned long long t;
  asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t) :: "memory");
  return t;
}
__device__ __forceinline__ void phase_set(int i, unsigned long long v) {
  // a wave-uniform condition, so that no scalar value becomes divergent
  if (__builtin_amdgcn_readfirstlane(threadIdx.x) < 64) {
    const int w = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    if (w < kTraceRows) {
      unsigned long long* row = g_phase_trace[w];
      if (i == 1) row[10] += 1;                        // a piece starts
      if (i == 9) row[9] = row[9] > v ? row[9] : v;    // merged in any piece
      else if (i == 0 || i == 8 || row[10] <= 1) row[i] = v;  // first piece, last end
    }
  }
}
#define PKV_PHASE(i) phase_set((i), phase_clock())
#define PKV_PHASE_VALUE(i, v) phase_set((i), (unsigned long long)(v))
#else
#define PKV_PHASE(i) do { } while (0)
#define PKV_PHASE_VALUE(i, v) do { } while (0)
#endif
