// Internal declarations shared by the host front (qgemv_host.cpp) and the
// kernels (qgemv_kernels.hip).  Not part of the C ABI.
#pragma once
#include <stdint.h>

#include "../../include/qgemv.h"

namespace qg {

// Work decomposition of one call (the wave64 counterpart of the pages' (L, R, S, K)
// tiles; M5 audit, section 2.1).  A wave covers two rows at a time with 32 lanes
// each; a lane owns 16 consecutive-in-layout weights of a 512-wide k slice.
struct Tile {
    int lanes_per_row;   // 32 (fixed by the kernels)
    int rows_per_batch;  // RB: rows each 32-lane group accumulates before a reduction (1,2,4,8)
    int waves_per_wg;    // NW: waves per workgroup; wave w takes k slices w, w+NW, ...
    int k_slice;         // 512 (fixed by the kernels)
    int rows_per_wg;     // RW: rows per workgroup (multiple of 2*RB)
    int mfma;            // 0: VALU path
};

constexpr int kLanesPerRow = 32;
constexpr int kWeightsPerLane = 16;
constexpr int kSlice = kLanesPerRow * kWeightsPerLane;  // 512
constexpr int kMaxWaves = 12;  // 768 threads: leaves 168 VGPRs per wave for x in registers

inline int pad_tokens(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : 4; }

// LDS of one workgroup: partial sums [batches][waves][2][rb * pad(T)] plus one
// arrival counter per batch.
inline size_t lds_bytes(const Tile& t, int T) {
    const size_t nbatch = (size_t)(t.rows_per_wg + 2 * t.rows_per_batch - 1) / (2 * t.rows_per_batch);
    return nbatch * t.waves_per_wg * 2 * t.rows_per_batch * pad_tokens(T) * 4 + nbatch * 4;
}
constexpr size_t kMaxLds = 64 * 1024;

inline bool valid_rb(int rb) { return rb == 1 || rb == 2 || rb == 4 || rb == 8; }

// The compiled set: rows_per_batch values instantiated for T tokens (the ones
// whose registers fit the 768-thread budget without spilling).  The grouped
// kernel serves up to 4 tokens per expert, so it uses the T = 4 row.
inline bool tile_supported(int T, int rb) {
    if (rb == 1 || rb == 2) return true;
    if (rb == 4) return T <= 3;
    if (rb == 8) return T == 1;
    return false;
}

struct DenseArgs {
    const uint8_t* W;
    const float* x;
    float* y;
    int64_t rows;
    int64_t row_bytes;
    int cols;
    int nslices;
    int rows_per_wg;
};

struct GroupedArgs {
    const uint8_t* W;
    const float* x;
    float* y;
    const int32_t* ids;
    int64_t rows;
    int64_t row_bytes;
    int64_t expert_bytes;
    int n_experts;
    int cols;
    int nslices;
    int rows_per_wg;
    int tiles_per_expert;
    int T;
    int topk;
};

// Launchers (qgemv_kernels.hip).  Return a hipError_t value as int.
int launch_dense(int fmt, int T, const Tile& tile, const DenseArgs& a, void* stream);
int launch_grouped(int fmt, const Tile& tile, const GroupedArgs& a, void* stream);
const char* hip_error_name(int err);

}  // namespace qg
