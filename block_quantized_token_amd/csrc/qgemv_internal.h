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
    int mfma;            // 1: streamed tiles contracted on the matrix cores (kind 1 only); 2: its persistent form
    int kind;            // 0: direct (lanes load their own bytes); 1: streamed through LDS via
                         // registers; 2: streamed by LDS-DMA loads into a ring of `depth` buffers,
                         // x staged in the ring's last slots; 3: as 2, x staged in its own region;
                         // 4: unit-balanced LDS-DMA (waves take equal shares of (slice, tile) units);
                         // 7: LDS-DMA on 256-wide k slices, 16 lanes per row; 8: matrix cores on
                         // 256-wide k slices fed by LDS-DMA loads of 16-row tiles; 9: persistent
                         // matrix cores on 512-wide slices fed by LDS-DMA loads; 11: kind 8 on
                         // 512-wide slices
    int depth;           // kinds 2, 3: tiles in flight per wave (2, 3, 4 or 6); kind 4: 2..4; kind 7: 2, 3; 0 otherwise
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
// (a workgroup of a single batch uses only the first nw * 2 * N floats)
// gfx950 gives one workgroup up to the CU's whole 160 KB of LDS.
constexpr size_t kMaxLds = 160 * 1024;

inline bool valid_rb(int rb) { return rb == 1 || rb == 2 || rb == 4 || rb == 8 || rb == 16; }

// The compiled set: rows_per_batch values instantiated for T tokens (the ones
// whose registers fit the 768-thread budget without spilling).  The grouped
// kernel serves up to 4 tokens per expert, so it uses the T = 4 row.
// A workgroup of one batch whose waves have one k slice each runs the one-shot
// kernel (every load of a wave in flight at once, one reduction); otherwise the
// pipelined kernel (ping-pong batches) runs.
inline bool one_shot(const Tile& t, int nslices) {
    return t.rows_per_wg == 2 * t.rows_per_batch && nslices <= t.waves_per_wg;
}

// Streamed kernel: a tile is 2 * RB rows; RB in {4, 8}.  Chunks (16 B) per full
// row slice and the per-wave LDS buffer it needs.
inline int stream_chunks(int fmt) { return fmt == QG_FMT_Q8_0 ? 34 : fmt == QG_FMT_Q4_0 ? 18 : 64; }
inline size_t stream_buf_bytes(int fmt, int rb) { return (size_t)((2 * rb * stream_chunks(fmt) + 63) / 64) * 1024; }
// waves_per_wg = nslices * row groups; each row group walks its tiles in pairs.
inline size_t stream_lds_bytes(int fmt, const Tile& t, int T, int nslices) {
    const size_t rg = (size_t)(t.waves_per_wg / nslices);
    size_t ntiles = (size_t)(t.rows_per_wg + 2 * t.rows_per_batch - 1) / (2 * t.rows_per_batch);
    ntiles = (ntiles + 2 * rg - 1) / (2 * rg) * (2 * rg);
    return t.waves_per_wg * stream_buf_bytes(fmt, t.rows_per_batch) +
           ntiles * nslices * 2 * t.rows_per_batch * pad_tokens(T) * 4;
}
inline bool stream_supported(int fmt, int T, int rb) {
    if (rb == 4) return fmt != QG_FMT_BF16 || T <= 2;
    if (rb == 8) return (fmt == QG_FMT_Q8_0 && T == 1) || (fmt == QG_FMT_Q4_0 && T <= 2);
    return false;
}

// LDS-DMA streamed kernel: 8-row tiles (rb 4), a ring of `depth` tile buffers per
// wave, partial sums [tiles][slices][2][rb * pad(T)] after the rings.
// x of the slice (T x 512 fp32) is staged in the last ring slots, so the depth
// must exceed the slots it takes.
inline int dma_x_slots(int fmt, int T) {
    const size_t buf = stream_buf_bytes(fmt, 4);
    return (int)((T * kSlice * 4 + buf - 1) / buf);
}
inline bool dma_supported(int fmt, int T, int rb, int depth, bool xsep) {
    return rb == 4 && (depth == 2 || depth == 3 || depth == 4 || depth == 6) && (xsep || dma_x_slots(fmt, T) < depth);
}
// rings, then (kind 3) x regions [waves][T][2 KB], then partial sums
inline size_t dma_lds_bytes(int fmt, const Tile& t, int T, int nslices) {
    const size_t ntiles = (size_t)(t.rows_per_wg + 2 * t.rows_per_batch - 1) / (2 * t.rows_per_batch);
    return (size_t)t.waves_per_wg * (t.depth * stream_buf_bytes(fmt, t.rows_per_batch) + (t.kind == 3 ? T * 2048 : 0)) +
           ntiles * nslices * 2 * t.rows_per_batch * pad_tokens(T) * 4;
}

// Half-slice LDS-DMA kernel (kind 7): 256-wide k slices (cols a multiple of 256),
// one wave per slice (times row groups), 8-row tiles (rb 4) in rings of `depth`
// (2 or 3) slots of 3 / 2 / 4 KB (Q8_0 / Q4_0 / BF16), x of the slice staged apart
// ([waves][T][1 KB]), then partial sums [tiles][slices][4 groups][2 rows * pad(T)].
inline bool half_supported(int rb, int depth) { return rb == 4 && (depth == 2 || depth == 3); }
inline size_t half_slot_bytes(int fmt) { return (size_t)((8 * (stream_chunks(fmt) / 2) + 63) / 64) * 1024; }
inline size_t half_lds_bytes(int fmt, const Tile& t, int T, int nslices256) {
    const size_t ntiles = (size_t)(t.rows_per_wg + 7) / 8;
    return (size_t)t.waves_per_wg * (t.depth * half_slot_bytes(fmt) + (size_t)T * 1024) +
           ntiles * nslices256 * 4 * 2 * pad_tokens(T) * 4;
}

// Kind 8 (matrix cores on 256-wide slices): one tile slot per wave (exactly the tile's
// bytes), a region per wave for one token's bf16 pieces (1536 bytes), then partial
// sums [tiles][slices][tile rows][pad(T)].
// `depth` is the tile's groups of 16 rows (1 or 2); kind 11 is kind 8 on 512-wide
// slices (two 256-wide halves, 16-row tiles), `nslices` the slices of its width.
inline size_t mx_slot_bytes(int fmt, int R = 1, int H = 1) {
    return (size_t)16 * R * (stream_chunks(fmt) / 2) * H * 16;
}
inline size_t mx_lds_bytes(int fmt, const Tile& t, int T, int nslices) {
    const int H = t.kind == 11 ? 2 : 1;
    const int R = t.depth == 2 && H == 1 ? 2 : 1;
    const size_t ntiles = (size_t)(t.rows_per_wg + 16 * R - 1) / (16 * R);
    return (size_t)t.waves_per_wg * (mx_slot_bytes(fmt, R, H) + 1536) + ntiles * nslices * 16 * R * pad_tokens(T) * 4;
}

// Kind 9 (persistent matrix cores on 512-wide slices): one 16-row tile slot per wave
// (the tile's bytes, at least 8 KB: x and its pieces are staged in it first), two chunk
// buffers of rows_per_wg / 16 tiles of partial sums [2][C][slices][16][pad(T)],
// four control words.
inline size_t mxp_slot_bytes(int fmt) {
    const size_t tile = (size_t)16 * stream_chunks(fmt) * 16;
    return tile > 8192 ? tile : 8192;
}
inline size_t mxp_lds_bytes(int fmt, const Tile& t, int T) {
    return (size_t)t.waves_per_wg * mxp_slot_bytes(fmt) +
           (size_t)2 * (t.rows_per_wg / 16) * t.waves_per_wg * 16 * pad_tokens(T) * 4 + 16;
}
// ... and, when it fits, the workgroup's outputs [T][ybuf_rows] after them
inline size_t mxp_ybuf_bytes(int64_t ybuf_rows, int T) { return (size_t)ybuf_rows * T * 4; }

// Row-subset kernel: rings of `depth` 8-row slots per wave, then partial sums (x in registers).
inline size_t gather_lds_bytes(int fmt, const Tile& t, int T, int nslices) {
    const size_t ntiles = (size_t)(t.rows_per_wg + 2 * t.rows_per_batch - 1) / (2 * t.rows_per_batch);
    return (size_t)t.waves_per_wg * t.depth * stream_buf_bytes(fmt, t.rows_per_batch) +
           ntiles * nslices * 2 * t.rows_per_batch * pad_tokens(T) * 4;
}

// Unit-balanced DMA kernel: x[T][cols] staged whole, then per-wave rings of
// `depth` 8-row tile slots, then partial sums.  Any number of waves.
inline bool units_supported(int rb, int depth) { return rb == 4 && depth >= 2 && depth <= 4; }
inline size_t units_lds_bytes(int fmt, const Tile& t, int T, int64_t cols) {
    const size_t nslices = (size_t)((cols + kSlice - 1) / kSlice);
    const size_t ntiles = (size_t)(t.rows_per_wg + 2 * t.rows_per_batch - 1) / (2 * t.rows_per_batch);
    return ((size_t)T * cols * 4 + 1023) / 1024 * 1024 +
           (size_t)t.waves_per_wg * t.depth * stream_buf_bytes(fmt, t.rows_per_batch) +
           ntiles * nslices * 2 * t.rows_per_batch * pad_tokens(T) * 4;
}

// Matrix-core streamed kernel: 16-row tiles (rb 8), Q8_0, any T.
inline bool mfma_supported(int fmt, int rb) { return fmt == QG_FMT_Q8_0 && rb == 8; }
// Its persistent form: one workgroup per CU (256 CUs), one wave per k slice;
// rows_per_wg is the chunk of rows whose partial sums are buffered (two chunks).
constexpr int kPersistGrid = 256;
inline size_t mfma_persist_lds_bytes(const Tile& t, int T) {
    const size_t chunk_tiles = (size_t)t.rows_per_wg / 16;
    return (size_t)t.waves_per_wg * stream_buf_bytes(QG_FMT_Q8_0, 8) +
           2 * chunk_tiles * t.waves_per_wg * 16 * pad_tokens(T) * 4 + 16;
}

inline bool tile_supported(int fmt, int T, int rb, bool oneshot) {
    if (!valid_rb(rb) || rb * pad_tokens(T) > 32) return false;
    if (oneshot) return true;
    if (rb == 1 || rb == 2) return true;
    if (rb == 4) return T <= 3;
    if (rb == 8) return T == 1 && fmt != QG_FMT_BF16;
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
    int ybuf_rows = 0;  // kind 9: rows of y a workgroup holds in LDS until its end (0: stores as it goes)
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
    const uint8_t* W2;  // parts == 2: the second table (up, beside gate in W), same shape
    float* y2;          // parts == 2: its outputs, [T][topk][rows]
    int parts;          // 1, or 2 (W and W2 in one launch)
    int per_slot_x;     // 0: x is [T][cols], one row per token; 1: [T][topk][cols], one per slot
};

// Launchers (qgemv_kernels.hip).  Return a hipError_t value as int.
int launch_dense(int fmt, int T, const Tile& tile, const DenseArgs& a, void* stream);
int launch_stream(int fmt, int T, const Tile& tile, const DenseArgs& a, void* stream);
int launch_dma(int fmt, int T, const Tile& tile, const DenseArgs& a, void* stream);
int launch_units(int fmt, int T, const Tile& tile, const DenseArgs& a, void* stream);
int launch_half(int fmt, int T, const Tile& tile, const DenseArgs& a, void* stream);
int launch_mx(int fmt, int T, const Tile& tile, const DenseArgs& a, void* stream);
int launch_mxp(int fmt, int T, const Tile& tile, const DenseArgs& a, void* stream);
// Fused argmax: fills work (uint64[T]), runs the mat-vec, writes idx/val (3 launches).
int launch_argmax(int fmt, int T, const Tile& tile, const DenseArgs& a, void* work, int32_t* idx, float* val,
                  void* stream);
int launch_grouped(int fmt, const Tile& tile, const GroupedArgs& a, void* stream);
// Row subset: y[t][i] = W[ids[i]] . x[t], i < nsel (kind-3 tile, rb 4, depth 2, rows_per_wg <= 64).
int launch_gather(int fmt, int T, const Tile& tile, const DenseArgs& a, const int32_t* ids, int64_t nsel, void* stream);
// Quantizers (qquant_kernels.hip): kind 0 Q8_0, 1 Q4_0 absmax, 2 Q4_0 Lloyd; nblocks
// blocks of 32 fp32 values in, as many packed blocks out.
int launch_quantize(int kind, const float* src, uint8_t* dst, int64_t nblocks, void* stream);
// HBM read probe (qprobe_kernels.hip): reads `bytes` (a multiple of 16) once, with
// at most max_groups workgroups of 256 lanes; stores to *out only in practice never.
int launch_read_probe(const void* src, int64_t bytes, int64_t max_groups, uint32_t magic, uint32_t* out,
                      void* stream);
const char* hip_error_name(int err);

// Keys of the allocation-free fused argmax (one per token) and the devices whose
// copy of them the library can address.
constexpr int kArgmaxScratchKeys = QG_MAX_T;
constexpr int kMaxDevices = 64;
// The current device's copy of the allocation-free argmax's keys (device memory of
// kArgmaxScratchKeys uint64 values, looked up once per device); 0 or a hipError_t.
int argmax_scratch(void** out);

}  // namespace qg
