// Host-side launch helpers shared by the kernel translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include "argreduce_device.hpp"

namespace argreduce {

// A fresh per-call nonce for the published words of a call; never 0 (the value words are
// reset to) nor 0xffffffff.
uint32_t next_nonce();

// Polls of one published word before a bounded wait gives up (argreduce_debug_set_spin_limit;
// default 2^20, about a second).
uint32_t spin_limit();
void set_spin_limit(uint32_t polls);  // 0 restores the default

// Copies the current device's count of look-back waits of the scan that gave up (synchronous).
hipError_t read_scan_wait_timeouts(unsigned long long* count);

// Measurement events (argreduce_debug_set_kernel_events); null when unset.
extern std::atomic<hipEvent_t> g_ev_start;
extern std::atomic<hipEvent_t> g_ev_stop;

// Launch of a scanning kernel (256-thread workgroups); with the measurement events set,
// the HIP extension launch records them around the kernel on the same stream.
template <typename... KArgs, typename... Args>
void launch_scan(void (*kernel)(KArgs...), dim3 grid, hipStream_t s, Args... args) {
    hipEvent_t e0 = g_ev_start.load(std::memory_order_relaxed);
    hipEvent_t e1 = g_ev_stop.load(std::memory_order_relaxed);
    if (e0 != nullptr && e1 != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, dim3(kBlockThreads), 0, s, e0, e1, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, dim3(kBlockThreads), 0, s, args...);
}

}  // namespace argreduce
