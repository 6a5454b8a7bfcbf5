// Streaming-read probe (measurement aid, include/pa_probe.h): reads a buffer
// once with the decode kernels' 16-byte loads, so a benchmark can quote the
// achievable HBM read rate beside the vendor peak.
#include <hip/hip_runtime.h>

#include "../../include/pa.h"
#include "../../include/pa_probe.h"
#include "pa_device.h"

namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeUnroll = 4;  // independent 16-byte loads in flight per lane

template <int NT>
__global__ __launch_bounds__(kProbeThreads) void hbm_read_probe_kernel(const uint4* __restrict__ src, int64_t n16,
                                                                       int64_t chunk16, uint32_t* __restrict__ sink,
                                                                       uint32_t magic, int scattered) {
    uint32_t acc = 0;
    if (chunk16 == 0) {
        // Grid-stride over 16-byte chunks: consecutive lanes read consecutive
        // chunks (1 KB per wavefront load), kProbeUnroll strides per iteration.
        const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads;
        int64_t i = static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
        for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
            uint4 v[kProbeUnroll];
#pragma unroll
            for (int u = 0; u < kProbeUnroll; ++u) v[u] = pa::load16<NT>(src + i + u * stride);
#pragma unroll
            for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
        for (; i < n16; i += stride) {
            const uint4 v = pa::load16<NT>(src + i);
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    } else {
        // Contiguous runs, as the decode kernels read whole K/V blocks:
        // workgroup w reads runs w, w + grid, w + 2 grid, ... of chunk16
        // 16-byte chunks each (a multiple of the workgroup's 512), lanes on
        // consecutive chunks, kProbeUnroll loads in flight per lane.
        // Scattered: the run index goes through the bijection r -> r *
        // 0x9E3779B1 mod nruns (an odd multiplier; nruns a power of two, host
        // check), so consecutive runs of a workgroup, and the runs read at
        // one time, lie at scattered addresses, as paged blocks do.
        const int64_t nruns = (n16 + chunk16 - 1) / chunk16;
        for (int64_t r = blockIdx.x; r < nruns; r += gridDim.x) {
            const int64_t rr = scattered ? ((r * int64_t{0x9E3779B1}) & (nruns - 1)) : r;
            const int64_t end = min(n16, (rr + 1) * chunk16);
            int64_t i = rr * chunk16 + threadIdx.x;
            for (; i + (kProbeUnroll - 1) * kProbeThreads < end; i += kProbeUnroll * kProbeThreads) {
                uint4 v[kProbeUnroll];
#pragma unroll
                for (int u = 0; u < kProbeUnroll; ++u) v[u] = pa::load16<NT>(src + i + u * kProbeThreads);
#pragma unroll
                for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
            }
            for (; i < end; i += kProbeThreads) {
                const uint4 v = pa::load16<NT>(src + i);
                acc ^= v.x ^ v.y ^ v.z ^ v.w;
            }
        }
    }
    // The data decide whether anything is written, so the loads stay; with
    // any magic value the data do not hit, nothing is.
    if (acc == magic) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" int pa_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t num_workgroups,
                                 size_t run_bytes, uint32_t magic, uint32_t flags, void* stream) {
    if (!src || !sink) return PA_ERR_NULL;
    if (bytes == 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(src) & 15u) || num_workgroups <= 0 ||
        num_workgroups > 65535 || run_bytes % (16 * kProbeThreads) ||
        (flags & ~static_cast<uint32_t>(PA_PROBE_NONTEMPORAL | PA_PROBE_SCATTERED)))
        return PA_ERR_INVALID;
    const int64_t n16 = static_cast<int64_t>(bytes / 16);
    const int64_t run16 = static_cast<int64_t>(run_bytes / 16);
    const int scattered = (flags & PA_PROBE_SCATTERED) ? 1 : 0;
    if (scattered) {
        // Whole runs only, and a power-of-two count of them (the bijection).
        if (run16 == 0 || n16 % run16) return PA_ERR_INVALID;
        const int64_t nruns = n16 / run16;
        if (nruns & (nruns - 1)) return PA_ERR_INVALID;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (flags & PA_PROBE_NONTEMPORAL)
        hipLaunchKernelGGL(hbm_read_probe_kernel<1>, dim3(num_workgroups), dim3(kProbeThreads), 0, s,
                           static_cast<const uint4*>(src), n16, run16, sink, magic, scattered);
    else
        hipLaunchKernelGGL(hbm_read_probe_kernel<0>, dim3(num_workgroups), dim3(kProbeThreads), 0, s,
                           static_cast<const uint4*>(src), n16, run16, sink, magic, scattered);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
