// On-device quantizers: fp32 [rows][cols] -> packed Q8_0 / Q4_0 blocks, in the
// layout the mat-vec kernels read (for gfx950, wave64).
//
// The pages name the quantizers and not their steps: Q4_0 draft weights come
// from the "Lloyd" quantizer of the hyper-connection loader (opus-mtp-turbo:
// Track 1 report, item 3 "Q4_0 / Q5_0 draft weights"), and dense projections
// are re-encoded to Q8_0 ("Where the time goes", meld-turbo-performance).
// Computed here, per block of 32 values, with every decision in fp32 one
// operation at a time (compiled with FMA contraction off):
//   Q8_0         d = max|v| / 127; code = round(v * (1/d)), halves away from 0.
//   Q4_0 absmax  the first element of largest magnitude, with its sign, is
//                mapped to code 0: d = that value / -8;
//                code = min(15, trunc(v * (1/d) + 8.5)).
//   Q4_0 Lloyd   from the absmax codes, alternately fit d by least squares,
//                d = sum v*q / sum q*q (q = code - 8, the sums in index order),
//                and move every code to the nearest level for that d,
//                clamp(floor(v * (1/d) + 8.5), 0, 15), until the codes stop
//                changing or 8 fits were made; the stored d is the last fit.
// The block stores fp16(d) (nearest, ties to even).  A block whose fp16 scale
// would be zero decodes to zeros whatever its codes, and is stored as the zero
// block (d = +0, codes 0 for Q8_0, 8 for Q4_0).  Non-finite inputs give
// unspecified bytes (never a fault).
//
// HBM-bound: 128 B read and 34 (18) B written per block.  A workgroup of 256
// lanes takes 256 consecutive blocks: coalesced 16-byte loads of its 32 KB into
// LDS (rows padded to 33 floats so that lane t's reads of block t do not
// collide on banks), one block per lane in registers, the packed bytes back
// through LDS and out as coalesced 16-byte stores (the workgroup's output is
// 8,704 or 4,608 contiguous, 16-byte-aligned bytes).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qgemv_internal.h"

namespace qg {
namespace {

constexpr int kQThreads = 256;  // lanes = blocks per workgroup
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kQStride = 33;    // floats per block row in LDS

__device__ __forceinline__ uint16_t fp16_bits(float d) {
    const _Float16 h = (_Float16)d;  // v_cvt_f16_f32: nearest, ties to even
    return __builtin_bit_cast(uint16_t, h);
}

template <int KIND>  // 0: Q8_0; 1: Q4_0 absmax; 2: Q4_0 Lloyd
__global__ void __launch_bounds__(kQThreads) quantize_kernel(const float* __restrict__ src, uint8_t* __restrict__ dst,
                                                             int64_t nblocks) {
    constexpr int OUT = KIND == 0 ? 34 : 18;
    __shared__ float xs[kQThreads * kQStride];
    __shared__ __attribute__((aligned(16))) uint8_t ob[kQThreads * OUT];
    const int t = threadIdx.x;
    const int64_t b0 = (int64_t)blockIdx.x * kQThreads;
    const int nb = nblocks - b0 < kQThreads ? (int)(nblocks - b0) : kQThreads;

    // 32 KB of input: 8 float4 per block, consecutive lanes on consecutive 16 B.
    // A full workgroup issues all 8 loads before it stores any (a bounds check
    // per load would make each one wait for the previous); the last, partial
    // workgroup checks each.
    const f32x4* s4 = reinterpret_cast<const f32x4*>(src + b0 * 32);
    auto put = [&](int idx, const f32x4& v) {
        float* p = xs + (idx >> 3) * kQStride + (idx & 7) * 4;
        p[0] = v.x;
        p[1] = v.y;
        p[2] = v.z;
        p[3] = v.w;
    };
    if (nb == kQThreads) {
        f32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __builtin_nontemporal_load(s4 + t + kQThreads * i);
#pragma unroll
        for (int i = 0; i < 8; ++i) put(t + kQThreads * i, v[i]);
    } else {
        for (int i = 0; i < 8; ++i) {
            const int idx = t + kQThreads * i;
            if (idx < nb * 8) put(idx, __builtin_nontemporal_load(s4 + idx));
        }
    }
    __syncthreads();

    if (t < nb) {
        float v[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) v[j] = xs[t * kQStride + j];
        uint16_t* o = reinterpret_cast<uint16_t*>(ob + t * OUT);  // t * OUT is even
        if constexpr (KIND == 0) {
            float amax = 0.0f;
#pragma unroll
            for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
            const float d = amax / 127.0f;
            uint16_t dh = fp16_bits(d);
            float id = 1.0f / d;
            if ((dh & 0x7FFF) == 0) {
                dh = 0;
                id = 0.0f;
            }
            o[0] = dh;
#pragma unroll
            for (int j = 0; j < 32; j += 2) {
                const int c0 = (int)__builtin_roundf(v[j] * id);
                const int c1 = (int)__builtin_roundf(v[j + 1] * id);
                o[1 + j / 2] = (uint16_t)((c0 & 0xFF) | ((c1 & 0xFF) << 8));
            }
        } else {
            float amax = 0.0f, vmax = 0.0f;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const float a = fabsf(v[j]);
                if (amax < a) {
                    amax = a;
                    vmax = v[j];
                }
            }
            float d = vmax / -8.0f;
            float id = 1.0f / d;
            if ((fp16_bits(d) & 0x7FFF) == 0) {
                d = 0.0f;
                id = 0.0f;
            }
            int c[32];
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                float s = v[j] * id;
                s = s + 8.5f;
                const int q = (int)s;
                c[j] = q < 15 ? q : 15;
            }
            if constexpr (KIND == 2) {
                for (int it = 0; it < 8; ++it) {
                    float s1 = 0.0f;
                    int s2 = 0;
#pragma unroll
                    for (int j = 0; j < 32; ++j) {
                        const int q = c[j] - 8;
                        s1 = s1 + v[j] * (float)q;
                        s2 += q * q;
                    }
                    if (s2 == 0) break;
                    d = s1 / (float)s2;
                    if (it == 7 || d == 0.0f) break;
                    const float idl = 1.0f / d;
                    bool changed = false;
#pragma unroll
                    for (int j = 0; j < 32; ++j) {
                        float s = v[j] * idl;
                        s = s + 8.5f;
                        s = floorf(s);
                        const int q = s < 0.0f ? 0 : s > 15.0f ? 15 : (int)s;
                        changed |= q != c[j];
                        c[j] = q;
                    }
                    if (!changed) break;
                }
            }
            o[0] = fp16_bits(d);
#pragma unroll
            for (int j = 0; j < 16; j += 2) {
                const int lo = c[j] | (c[j + 16] << 4), hi = c[j + 1] | (c[j + 17] << 4);
                o[1 + j / 2] = (uint16_t)(lo | (hi << 8));
            }
        }
    }
    __syncthreads();

    uint8_t* out = dst + b0 * OUT;  // 16-byte aligned: b0 * OUT is a multiple of 4,608
    if (nb == kQThreads) {
        constexpr int N16 = kQThreads * OUT / 16;
        for (int i = t; i < N16; i += kQThreads)
            reinterpret_cast<uint4*>(out)[i] = reinterpret_cast<const uint4*>(ob)[i];
    } else {
        const int n2 = nb * OUT / 2;
        for (int i = t; i < n2; i += kQThreads)
            reinterpret_cast<uint16_t*>(out)[i] = reinterpret_cast<const uint16_t*>(ob)[i];
    }
}

}  // namespace

int launch_quantize(int kind, const float* src, uint8_t* dst, int64_t nblocks, void* stream) {
    const unsigned grid = (unsigned)((nblocks + kQThreads - 1) / kQThreads);
    auto fn = kind == 0 ? quantize_kernel<0> : kind == 1 ? quantize_kernel<1> : quantize_kernel<2>;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(kQThreads), 0, (hipStream_t)stream, src, dst, nblocks);
    return (int)hipGetLastError();
}

}  // namespace qg
