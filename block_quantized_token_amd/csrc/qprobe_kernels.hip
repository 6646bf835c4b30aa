// HBM read probe (gfx950): reads a buffer once with coalesced 16-byte
// non-temporal loads and nothing else, so that the mat-vec's effective
// bandwidth can be set beside what a plain streaming read of the same bytes
// achieves on this part (the measurement the M2 Max page takes as its peak
// reference: "Where the time goes on an M2 Max", the bandwidth the mat-vec
// table is compared against).
//
// Each lane keeps kLoads loads of 16 bytes in flight per step of a grid-stride
// loop over the buffer and folds what it read into one word by XOR; a wave
// whose word equals the caller's `magic` stores it, so the loads cannot be
// dropped and nothing else is written in practice.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qgemv_internal.h"

namespace qg {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeLoads = 8;  // 16-byte loads in flight per lane per step
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kProbeThreads)
read_probe_kernel(const u32x4* __restrict__ src, int64_t n16, uint32_t magic, uint32_t* out) {
    uint32_t acc = 0;
    const int64_t step = (int64_t)gridDim.x * kProbeThreads * kProbeLoads;
    for (int64_t base = (int64_t)blockIdx.x * kProbeThreads * kProbeLoads + threadIdx.x; base < n16; base += step) {
        u32x4 v[kProbeLoads];
#pragma unroll
        for (int u = 0; u < kProbeLoads; ++u) {
            const int64_t i = base + (int64_t)u * kProbeThreads;
            v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kProbeLoads; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == magic) *out = acc;
}

}  // namespace

int launch_read_probe(const void* src, int64_t bytes, int64_t max_groups, uint32_t magic, uint32_t* out,
                      void* stream) {
    const int64_t n16 = bytes / 16;
    const int64_t per_group = (int64_t)kProbeThreads * kProbeLoads;
    int64_t grid = (n16 + per_group - 1) / per_group;
    grid = grid < max_groups ? grid : max_groups;
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, (hipStream_t)stream,
                       (const u32x4*)src, n16, magic, out);
    return (int)hipGetLastError();
}

}  // namespace qg
