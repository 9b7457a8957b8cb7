// Phase stamps for kernel timelines.  Compiled in only when MONO_TRACE is
// defined (the separate trace library, libmono_decode_trace.so); in the
// product library every macro below expands to nothing.
//
// Thread 0 of a workgroup writes the 100 MHz device clock (s_memrealtime)
// into records of kTraceStamps words:
//   item records (one per work item, indexed by the item's ticket):
//     stamp 0 = item start, 1 = item end, 2..30 = phases of the item kind
//     (see the MONO_STAMP calls: 2..9 scan and selection phases, 10..16
//     attention, 17 a whole selection), word 31 = (kind << 24) | item index;
//   workgroup records (one per workgroup): stamp 0 = kernel entry, 1 = exit.
// A stamp is a global store, so the trace build runs a little slower than
// the product build (its waits for memory also wait for the stamps).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mono {

constexpr int kTraceItems = 8192;   // item records kept (later tickets are not recorded)
constexpr int kTraceGroups = 4096;  // workgroup records kept
constexpr int kTraceStamps = 32;    // words per record
constexpr uint32_t kTraceClearKind = 0xFFu;  // the kind word of a clear item

#ifdef MONO_TRACE
extern __device__ uint64_t g_trace_items[kTraceItems * kTraceStamps];
extern __device__ uint64_t g_trace_groups[kTraceGroups * kTraceStamps];

// The record of the item this workgroup runs (thread 0's copy is the one used).
__device__ __forceinline__ uint32_t& trace_record() {
  __shared__ uint32_t rec;
  return rec;
}

#define MONO_TRACE_ITEM(ticket, note)                                                      \
  do {                                                                                     \
    if (threadIdx.x == 0) {                                                                \
      ::mono::trace_record() = (uint32_t)(ticket);                                         \
      if ((uint32_t)(ticket) < (uint32_t)::mono::kTraceItems) {                            \
        ::mono::g_trace_items[(size_t)(ticket) * ::mono::kTraceStamps + 31] = (note);      \
        ::mono::g_trace_items[(size_t)(ticket) * ::mono::kTraceStamps] = wall_clock64();   \
      }                                                                                    \
    }                                                                                      \
  } while (0)
#define MONO_STAMP(k)                                                                              \
  do {                                                                                             \
    if (threadIdx.x == 0 && ::mono::trace_record() < (uint32_t)::mono::kTraceItems)                \
      ::mono::g_trace_items[(size_t)::mono::trace_record() * ::mono::kTraceStamps + (k)] = wall_clock64(); \
  } while (0)
#define MONO_STAMP_GROUP(k)                                                                    \
  do {                                                                                         \
    if (threadIdx.x == 0 && blockIdx.x < (uint32_t)::mono::kTraceGroups)                       \
      ::mono::g_trace_groups[(size_t)blockIdx.x * ::mono::kTraceStamps + (k)] = wall_clock64(); \
  } while (0)
#else
#define MONO_TRACE_ITEM(ticket, note) \
  do {                                \
  } while (0)
#define MONO_STAMP(k) \
  do {                \
  } while (0)
#define MONO_STAMP_GROUP(k) \
  do {                      \
  } while (0)
#endif

}  // namespace mono
