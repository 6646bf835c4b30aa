// HIP kernels (gfx950) for the multi-token block-quantized mat-vec
//     y[t][r] = sum_k w[r][k] * x[t][k],  t < T <= 4,
// the product the M5 multi-token audit ("Track 2 Audit & Optimization Report: M5
// Metal Kernels for Multi-Token Speculative Decode") tunes in section 2.1 and the
// M2 Max page ("Where the time goes on an M2 Max") measures in its mat-vec table.
//
// Work mapping (wave64, re-derived for CDNA4 rather than taken from the pages'
// simdgroup tiles):
//   * a k slice is 512 weights: 16 Q8_0/Q4_0 blocks or 512 bf16 values;
//   * a wave works on two rows at once, 32 lanes per row; lane li of a row owns
//     16 weights of the slice (half a block for Q8_0/Q4_0), so the slice's
//     activations x[t][k] live in that lane's registers for every row it visits
//     -- each decoded weight is reused across all T tokens straight from
//     registers, and x never goes through LDS in the hot loop;
//   * per row and lane the weight bytes come in with one 16-byte load (Q8_0: the
//     lane's 16 codes; Q4_0: 8 bytes; BF16: two 16-byte loads) plus the block's
//     fp16 scale; the 32 lanes of a row cover 544 (Q8_0) / 288 (Q4_0) / 1024
//     (BF16) contiguous bytes, so every load instruction is coalesced;
//   * codes are decoded in registers (Q8_0: sign-extended bytes; Q4_0: nibbles
//     re-biased to signed and shifted into the top of a byte, with the factor 16
//     moved into the scale; BF16: a shift), multiplied by x in an fp32 fma chain
//     per token, and scaled once per block and token;
//   * the 32 lanes of a row reduce their partials with a halving butterfly
//     (each stage halves the number of live values per lane), then the waves of
//     the workgroup -- which split k -- add their partials through LDS in wave
//     order.
// Every output's summation order depends only on cols and the number of waves,
// never on T, so a token's result is the same bit for bit at any T (the pages
// remark on that property: opus-mtp-turbo report, finding 3).
#include <hip/hip_runtime.h>
#include <cstdlib>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "qgemv_internal.h"

// The allocation-free fused argmax keeps its per-token 64-bit keys here instead of
// in a caller-owned workspace: QG_MAX_T of them (32 bytes), one copy per GPU the
// library runs on, held until the process ends.  Host code never uses this name as
// an address (on the host it is only a stand-in for the device symbol): it passes
// the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned long long scratch[qg::kArgmaxScratchKeys];

namespace qg {
namespace {

struct __attribute__((packed, aligned(2))) U4u { uint32_t v[4]; };  // 16 B at 2-byte alignment
struct __attribute__((packed, aligned(2))) U2u { uint32_t v[2]; };  // 8 B at 2-byte alignment
struct __attribute__((aligned(16))) U4a { uint32_t v[4]; };
typedef uint32_t V4 __attribute__((ext_vector_type(4)));  // 16 B in four VGPRs

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// ---------------------------------------------------------------- formats
// Each format says which k positions lane li owns inside a 512-wide slice, where
// the lane's bytes of one row sit, and how to turn them into 16 fp32 weights (up
// to a per-block scale).  Loads are never predicated: a lane with no weights in
// range reads lane 0's bytes of the same row (always in range) and its result
// is dropped by a select, so every load of a batch can be in flight at once.
template <int FMT> struct Fmt;

template <> struct Fmt<QG_FMT_Q8_0> {
    static constexpr int kBlockBytes = 34;
    static constexpr bool kScaled = true;
    struct Raw { uint32_t c[4]; uint32_t d; };
    // block q = li / 2 of the slice, codes [16 h, 16 h + 16) with h = li % 2
    __device__ static int kbase(int li, int half) { return 32 * (li >> 1) + 16 * (li & 1) + 8 * half; }
    __device__ static int64_t slice_offset(int s) { return (int64_t)s * 16 * kBlockBytes; }
    __device__ static bool lane_valid(int li, int k0, int cols) { return k0 + 32 * (li >> 1) < cols; }
    __device__ static bool upper_valid(int, int, int) { return true; }
    __device__ static Raw load(const uint8_t* slice, int li) {
        const uint8_t* blk = slice + (li >> 1) * kBlockBytes;
        const U4u q = *reinterpret_cast<const U4u*>(blk + 2 + 16 * (li & 1));
        Raw r;
        r.c[0] = q.v[0]; r.c[1] = q.v[1]; r.c[2] = q.v[2]; r.c[3] = q.v[3];
        r.d = *reinterpret_cast<const uint16_t*>(blk);
        return r;
    }
    __device__ static float scale(const Raw& r) { return half_bits_to_float(r.d); }
    __device__ static float weight(const Raw& r, int i) {
        return (float)(int32_t)(int8_t)(r.c[i >> 2] >> (8 * (i & 3)));
    }
};

template <> struct Fmt<QG_FMT_Q4_0> {
    static constexpr int kBlockBytes = 18;
    static constexpr bool kScaled = true;
    struct Raw { uint32_t c[2]; uint32_t d; };
    // block q = li / 2, bytes [8 h, 8 h + 8) of its 16 code bytes: low nibbles are
    // codes 8h .. 8h+7 (weights 0..7), high nibbles codes 16 + 8h .. (weights 8..15)
    __device__ static int kbase(int li, int half) { return 32 * (li >> 1) + 8 * (li & 1) + 16 * half; }
    __device__ static int64_t slice_offset(int s) { return (int64_t)s * 16 * kBlockBytes; }
    __device__ static bool lane_valid(int li, int k0, int cols) { return k0 + 32 * (li >> 1) < cols; }
    __device__ static bool upper_valid(int, int, int) { return true; }
    __device__ static Raw load(const uint8_t* slice, int li) {
        const uint8_t* blk = slice + (li >> 1) * kBlockBytes;
        const U2u q = *reinterpret_cast<const U2u*>(blk + 2 + 8 * (li & 1));
        Raw r;
        r.c[0] = q.v[0]; r.c[1] = q.v[1];
        r.d = *reinterpret_cast<const uint16_t*>(blk);
        return r;
    }
    // codes are returned as 16 * (c - 8): flipping bit 3 of a nibble gives the
    // 4-bit two's complement of c - 8, and shifting it to the top of a byte makes
    // a signed byte; the 16 is taken back out of the scale (exact: a power of 2).
    __device__ static float scale(const Raw& r) { return half_bits_to_float(r.d) * 0.0625f; }
    __device__ static float weight(const Raw& r, int i) {
        const uint32_t w = r.c[(i & 7) >> 2] ^ 0x88888888u;
        const uint32_t b = (i < 8) ? (w << 4) : w;  // nibble to the top of its byte
        return (float)(int32_t)(int8_t)((b >> (8 * (i & 3))) & 0xF0u);
    }
};

template <> struct Fmt<QG_FMT_BF16> {
    static constexpr bool kScaled = false;
    struct Raw { uint32_t c[8]; };
    // values [16 li, 16 li + 16) of the slice
    __device__ static int kbase(int li, int half) { return 16 * li + 8 * half; }
    __device__ static int64_t slice_offset(int s) { return (int64_t)s * kSlice * 2; }
    __device__ static bool lane_valid(int li, int k0, int cols) { return k0 + 16 * li < cols; }
    // cols % 8 == 0: the lane's second 8 values may lie past the end of the row
    __device__ static bool upper_valid(int li, int k0, int cols) { return k0 + 16 * li + 8 < cols; }
    __device__ static Raw load(const uint8_t* slice, int li, bool upper_ok) {
        const U4a* p = reinterpret_cast<const U4a*>(slice + 32 * li);
        const U4a a = p[0];
        const U4a b = p[upper_ok ? 1 : 0];
        Raw r;
        r.c[0] = a.v[0]; r.c[1] = a.v[1]; r.c[2] = a.v[2]; r.c[3] = a.v[3];
        r.c[4] = b.v[0]; r.c[5] = b.v[1]; r.c[6] = b.v[2]; r.c[7] = b.v[3];
        return r;
    }
    __device__ static float scale(const Raw&) { return 1.0f; }
    __device__ static float weight(const Raw& r, int i) {
        const uint32_t w = r.c[i >> 1];
        return __builtin_bit_cast(float, (i & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
};

template <int FMT>
__device__ __forceinline__ typename Fmt<FMT>::Raw load_lane(const uint8_t* slice, int li_eff, bool upper_ok) {
    if constexpr (FMT == QG_FMT_BF16) return Fmt<FMT>::load(slice, li_eff, upper_ok);
    else return Fmt<FMT>::load(slice, li_eff);
}

// ------------------------------------------------------------- reduction
// Halving butterfly over the 32 lanes of a row: with N values per lane, stage m
// (16, 8, 4, 2, 1) pairs each lane with a partner whose lane bit m differs; the
// lane with bit m set keeps the upper half of its values and adds its partner's
// upper half, the other keeps the lower half.  After 5 stages value v's sum
// over all 32 lanes sits in the lanes whose index() is v.
//   stage 16: v_permlane16_swap (rows of 16 lanes swap halves; one add finishes)
//   stage  8: DPP row_mirror      (lane i <-> 15 - i)
//   stage  4: DPP row_half_mirror (lane i <-> 7 - i)
//   stage  2: DPP quad_perm [2,3,0,1]
//   stage  1: DPP quad_perm [1,0,3,2]
// The partner of a lane at each stage -- hence every value's addition tree --
// does not depend on N, so a token's sum does not depend on T.
__device__ __forceinline__ float dpp_f(float v, int ctrl) {
    switch (ctrl) {  // the control must be an immediate
    case 0x140: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
    case 0x141: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
    case 0x4E: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
    default: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
    }
}

// v_permlane16_swap a, b: lanes 16..31 of a trade places with lanes 0..15 of b
// (and 48..63 of a with 32..47 of b).  Written as inline asm with both operands
// read-write: the clang builtin of this ROCm release returns the first result
// twice (r[0] + r[1] compiles to v + v), so its second result cannot be used.
__device__ __forceinline__ void permlane16_swap(float& a, float& b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// v_permlane32_swap: a lane of the lower half ends with (its a, the a of lane + 32),
// a lane of the upper half with (the b of lane - 32, its b).
__device__ __forceinline__ void permlane32_swap(float& a, float& b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

template <int N>
__device__ __forceinline__ void butterfly32(float (&v)[N], int li) {
    // stage 16: after the swap, a lane of row 0 holds (its a, row 1's a) and a lane
    // of row 1 holds (row 0's b, its b): one add gives the lower / upper half sums
    if constexpr (N >= 2) {
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            float a = v[i], b = v[i + N / 2];
            permlane16_swap(a, b);
            v[i] = a + b;
        }
    } else {
        float a = v[0], b = v[0];
        permlane16_swap(a, b);
        v[0] = a + b;
    }
    constexpr int ctrls[4] = {0x140, 0x141, 0x4E, 0xB1};
#pragma unroll
    for (int st = 1; st < 5; ++st) {
        const int m = 16 >> st;
        const int cnt = N >> st;
        if (cnt >= 2) {
            const bool up = (li & m) != 0;
#pragma unroll
            for (int i = 0; i < cnt / 2; ++i) {
                const float lo = v[i] + dpp_f(v[i], ctrls[st - 1]);
                const float hi = v[i + cnt / 2] + dpp_f(v[i + cnt / 2], ctrls[st - 1]);
                v[i] = up ? hi : lo;
            }
        } else {
            v[0] = v[0] + dpp_f(v[0], ctrls[st - 1]);
        }
    }
}

template <int N>
__device__ __forceinline__ int butterfly_index(int li, bool& writer) {
    int idx = 0;
    writer = true;
#pragma unroll
    for (int st = 0; st < 5; ++st) {
        const int m = 16 >> st;
        const int cnt = N >> st;
        if (cnt >= 2) {
            if (li & m) idx += cnt / 2;
        } else if (li & m) {
            writer = false;
        }
    }
    return idx;
}

constexpr int pad_pow2(int t) { return t <= 1 ? 1 : t <= 2 ? 2 : 4; }

// ------------------------------------------------------------------ body
// One workgroup: rows [row_begin, row_end) of one matrix, all of k.  NT tokens;
// token n reads x + xoff[n] and its outputs go through out(n, row, value).
//
// A batch is 2*RB rows: each 32-lane half of a wave takes every other row.  The
// loads of batch b+1 are issued before batch b is computed (ping-pong register
// sets), so a wave always has a batch of weights in flight.
//
// Cross-wave reduction without barriers: every batch has its own LDS slots
// [wave][row group][value] and an arrival counter.  A wave writes its butterfly
// results, then bumps the counter; the wave that arrives last adds the NW
// partial sets in wave order and stores the outputs.  No wave ever waits for
// another, and no slot is reused within a launch.
template <int FMT, int NT, int RB>
struct RowsCtx {
    using F = Fmt<FMT>;
    static constexpr int TP = pad_pow2(NT);
    static constexpr int N = RB * TP;  // values per lane entering the butterfly
    const uint8_t* W;
    int64_t row_bytes, row_begin, row_end;
    int g, li;
};

template <int FMT, int NT, int RB>
__device__ __forceinline__ void issue_batch(const RowsCtx<FMT, NT, RB>& c, int64_t rb0, int64_t slice_off, int li_eff,
                                            bool upper_ok, typename Fmt<FMT>::Raw (&raw)[RB]) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        int64_t row = rb0 + 2 * r + c.g;
        row = row < c.row_end ? row : c.row_begin;  // out-of-range rows reread a valid row; never stored
        raw[r] = load_lane<FMT>(c.W + row * c.row_bytes + slice_off, li_eff, upper_ok);
    }
}

template <int FMT, int NT, int RB>
__device__ __forceinline__ void accumulate_batch(const typename Fmt<FMT>::Raw (&raw)[RB], const float (&xr)[NT][kWeightsPerLane],
                                                 bool lane_ok, bool upper_ok, float (&acc)[RB][pad_pow2(NT)]) {
    using F = Fmt<FMT>;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        float p[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) p[n] = 0.0f;
        float ph[NT];
#pragma unroll
        for (int i = 0; i < kWeightsPerLane; ++i) {
            if (i == kWeightsPerLane / 2) {
#pragma unroll
                for (int n = 0; n < NT; ++n) ph[n] = p[n];
            }
            const float w = F::weight(raw[r], i);
#pragma unroll
            for (int n = 0; n < NT; ++n) p[n] = __builtin_fmaf(w, xr[n][i], p[n]);
        }
        if constexpr (F::kScaled) {
            // a lane with nothing in range decoded finite codes from in-range bytes and
            // read in-range x, so its p is finite and 0 * p adds exactly nothing
            const float d = lane_ok ? F::scale(raw[r]) : 0.0f;
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[r][n] = __builtin_fmaf(d, p[n], acc[r][n]);
        } else {
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const float q = upper_ok ? p[n] : ph[n];  // drop values past the end of the row
                acc[r][n] = acc[r][n] + (lane_ok ? q : 0.0f);
            }
        }
    }
}

template <int FMT, int NT>
__device__ __forceinline__ void load_x(const float* __restrict__ x, const int64_t (&xoff)[NT], int k0, int li, bool lane_ok,
                                       int cols, float (&xr)[NT][kWeightsPerLane]) {
    using F = Fmt<FMT>;
    // two runs of 8 consecutive k per lane; a lane with nothing in range reads the
    // token's first 8 values (cols >= 8 always), and its products are discarded
    const int b0 = lane_ok ? k0 + F::kbase(li, 0) : 0;
    const int b1 = lane_ok ? k0 + F::kbase(li, 1) : 0;
    const int b1c = b1 + 8 <= cols ? b1 : b0;  // BF16 tail: the upper run may not exist
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const float4* p0 = reinterpret_cast<const float4*>(x + xoff[n] + b0);
        const float4* p1 = reinterpret_cast<const float4*>(x + xoff[n] + b1c);
        const float4 a = p0[0], b = p0[1], c = p1[0], d = p1[1];
        xr[n][0] = a.x; xr[n][1] = a.y; xr[n][2] = a.z; xr[n][3] = a.w;
        xr[n][4] = b.x; xr[n][5] = b.y; xr[n][6] = b.z; xr[n][7] = b.w;
        xr[n][8] = c.x; xr[n][9] = c.y; xr[n][10] = c.z; xr[n][11] = c.w;
        xr[n][12] = d.x; xr[n][13] = d.y; xr[n][14] = d.z; xr[n][15] = d.w;
    }
}


// Ordering for the arrival protocols, whose partial sums and counters live in LDS
// and move only through ds_ instructions.  A wave's LDS operations execute in order
// and the LDS atomics are serialized, so a release needs this wave's LDS accesses
// complete (lgkmcnt 0) and an acquire needs none; the asm barriers keep the
// compiler from moving LDS accesses across.  Unlike a fence, neither waits for the
// wave's loads into LDS in flight (the next tile), which the protocols never read.
__device__ __forceinline__ void lds_release() {
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void lds_acquire() { asm volatile("" ::: "memory"); }

template <int FMT, int NT, int RB, class Out>
__device__ __forceinline__ void reduce_batch(float (&acc)[RB][pad_pow2(NT)], int b, int64_t rb0, float* part,
                                             int* arrivals, int nw, int wave, int lane, int li, int g, int my_idx,
                                             bool writer, int64_t row_end, Out& out) {
    constexpr int TP = pad_pow2(NT);
    constexpr int N = RB * TP;
    float v[N];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < TP; ++t) v[r * TP + t] = acc[r][t];
    butterfly32<N>(v, li);
    float* mine = part + (((size_t)b * nw + wave) * 2 + g) * N;
    if (writer) mine[my_idx] = v[0];
    // publish this wave's slots, then count the arrival (one atomic per wave); the
    // slots and the counter are in LDS: the wave does not wait here for its loads in
    // flight
    lds_release();
    int prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(&arrivals[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    prev = __shfl(prev, 0, 64);
    if (prev == nw - 1) {  // last arrival: all nw partial sets of batch b are in LDS
        lds_acquire();
        if (lane < 2 * N) {
            const int gg = lane / N, idx = lane % N;
            const int t = idx % TP, r = idx / TP;
            const int64_t row = rb0 + 2 * r + gg;
            if (t < NT && row < row_end) {
                const float* base = part + (size_t)b * nw * 2 * N + gg * N + idx;
                float sum = base[0];
                for (int w = 1; w < nw; ++w) sum = sum + base[(size_t)w * 2 * N];
                out(t, row, sum);
            }
        }
    }
}

template <int FMT, int NT, int RB, bool ONE_SHOT, class Out>
__device__ __forceinline__ void gemv_rows(const uint8_t* __restrict__ W, int64_t row_bytes, int cols, int nslices,
                                          const float* __restrict__ x, const int64_t (&xoff)[NT], int64_t row_begin,
                                          int64_t row_end, int nw, Out&& out) {
    using F = Fmt<FMT>;
    using Raw = typename F::Raw;
    constexpr int TP = pad_pow2(NT);
    constexpr int N = RB * TP;
    static_assert(N <= 32, "rows_per_batch * tokens too large");
    extern __shared__ float lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps buffer descriptors scalar
    // nw: waves per workgroup, an argument
    const int g = lane >> 5;   // which of the two rows of a step
    const int li = lane & 31;  // lane within the row
    const int nbatch = (int)((row_end - row_begin + 2 * RB - 1) / (2 * RB));

    bool writer;
    const int my_idx = butterfly_index<N>(li, writer);
    const RowsCtx<FMT, NT, RB> c{W, row_bytes, row_begin, row_end, g, li};
    float xr[NT][kWeightsPerLane];
    float acc[RB][TP];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < TP; ++t) acc[r][t] = 0.0f;

    if constexpr (ONE_SHOT) {
        // One shot (the host guarantees one batch per workgroup and one slice
        // per wave): all of the wave's loads go out together, then one reduction
        // through LDS.  (A wave past the last slice would read slice 0 with
        // every lane invalid: it only adds zeros.)
        (void)nbatch;
        const int s = wave < nslices ? wave : 0;
        const int k0 = s * kSlice;
        const bool lane_ok = wave < nslices && F::lane_valid(li, k0, cols);
        const bool upper_ok = lane_ok && F::upper_valid(li, k0, cols);
        Raw ra[RB];
        issue_batch(c, row_begin, F::slice_offset(s), lane_ok ? li : 0, upper_ok, ra);
        load_x<FMT, NT>(x, xoff, k0, li, lane_ok, cols, xr);
        // every load is issued before the first use of any: otherwise the
        // scheduler may pull an early decode up to just after its load and
        // make the wave wait for it before issuing the rest (not for the
        // widest batches, whose registers would then spill)
        if constexpr (sizeof(Raw) * RB <= 256) __builtin_amdgcn_sched_barrier(0);
        accumulate_batch<FMT, NT, RB>(ra, xr, lane_ok, upper_ok, acc);
        float v[N];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int t = 0; t < TP; ++t) v[r * TP + t] = acc[r][t];
        butterfly32<N>(v, li);
        float* part = lds;  // [nw][2][N]
        if (writer) part[(wave * 2 + g) * N + my_idx] = v[0];
        __syncthreads();
        if (tid < 2 * N) {
            const int gg = tid / N, idx = tid % N;
            const int t = idx % TP, r = idx / TP;
            const int64_t row = row_begin + 2 * r + gg;
            if (t < NT && row < row_end) {
                const float* base = part + gg * N + idx;
                float sum = base[0];
                for (int w = 1; w < nw; ++w) sum = sum + base[w * 2 * N];
                out(t, row, sum);
            }
        }
        return;
    } else {

    float* part = lds;                                                           // [nbatch][nw][2][N]
    int* arrivals = reinterpret_cast<int*>(lds + (size_t)nbatch * nw * 2 * N);  // [nbatch]
    for (int i = tid; i < nbatch; i += blockDim.x) arrivals[i] = 0;
    __syncthreads();

    if (nslices <= nw) {
        // one slice per wave: x stays in registers; batch b+1 loads while b computes
        const int s = wave < nslices ? wave : 0;  // (a wave past the last slice only adds zeros)
        const int k0 = s * kSlice;
        const bool lane_ok = wave < nslices && F::lane_valid(li, k0, cols);
        const bool upper_ok = lane_ok && F::upper_valid(li, k0, cols);
        const int li_eff = lane_ok ? li : 0;
        const int64_t soff = F::slice_offset(s);
        Raw ra[RB], rb[RB];
        issue_batch(c, row_begin, soff, li_eff, upper_ok, ra);
        load_x<FMT, NT>(x, xoff, k0, li, lane_ok, cols, xr);
        for (int b = 0; b < nbatch; b += 2) {
            const int64_t r0 = row_begin + (int64_t)b * 2 * RB;
            // next batch (past the end: rows clamp to valid ones and nothing is stored)
            issue_batch(c, r0 + 2 * RB, soff, li_eff, upper_ok, rb);
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int t = 0; t < TP; ++t) acc[r][t] = 0.0f;
            accumulate_batch<FMT, NT, RB>(ra, xr, lane_ok, upper_ok, acc);
            reduce_batch<FMT, NT, RB>(acc, b, r0, part, arrivals, nw, wave, lane, li, g, my_idx, writer, row_end, out);
            if (b + 1 >= nbatch) break;
            issue_batch(c, r0 + 4 * RB, soff, li_eff, upper_ok, ra);
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int t = 0; t < TP; ++t) acc[r][t] = 0.0f;
            accumulate_batch<FMT, NT, RB>(rb, xr, lane_ok, upper_ok, acc);
            reduce_batch<FMT, NT, RB>(acc, b + 1, r0 + 2 * RB, part, arrivals, nw, wave, lane, li, g, my_idx, writer,
                                      row_end, out);
        }
        return;
    }

    // several slices per wave (cols > 512 * nw): x is reloaded per slice visit
    int loaded_slice = -1;
    bool lane_ok = false, upper_ok = false;
    for (int b = 0; b < nbatch; ++b) {
        const int64_t r0 = row_begin + (int64_t)b * 2 * RB;
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int t = 0; t < TP; ++t) acc[r][t] = 0.0f;
        for (int s = wave; s < nslices; s += nw) {
            const int k0 = s * kSlice;
            lane_ok = F::lane_valid(li, k0, cols);
            upper_ok = lane_ok && F::upper_valid(li, k0, cols);
            Raw ra[RB];
            issue_batch(c, r0, F::slice_offset(s), lane_ok ? li : 0, upper_ok, ra);
            if (s != loaded_slice) {
                load_x<FMT, NT>(x, xoff, k0, li, lane_ok, cols, xr);
                loaded_slice = s;
            }
            accumulate_batch<FMT, NT, RB>(ra, xr, lane_ok, upper_ok, acc);
        }
        reduce_batch<FMT, NT, RB>(acc, b, r0, part, arrivals, nw, wave, lane, li, g, my_idx, writer, row_end, out);
    }
    }
}

// ------------------------------------------------------- streamed variant
// For rows whose byte length is a multiple of 16 (Q8_0/Q4_0: cols % 256 == 0;
// BF16: cols % 8 == 0) and one k slice per wave.  Each wave streams its own
// slice of a tile of ST rows: the slice bytes of the tile are cut into aligned
// 16-byte chunks, lane l of load k fetching chunk 64k + l -- so every load
// instruction reads ~1 KB of contiguous row bytes -- into registers; the wave
// then writes them to its private LDS buffer in the same order and reads back
// its own lane's bytes (a block-aligned 16 / 8 / 32 bytes at an arbitrary LDS
// offset).  Two tiles are in flight per wave (ping-pong register sets); waves
// never wait for each other until one barrier before the final cross-wave sum.
template <int FMT> struct StreamFmt;
template <> struct StreamFmt<QG_FMT_Q8_0> { static constexpr int kChunks = 34; };  // 16 blocks x 34 B
template <> struct StreamFmt<QG_FMT_Q4_0> { static constexpr int kChunks = 18; };  // 16 blocks x 18 B
template <> struct StreamFmt<QG_FMT_BF16> { static constexpr int kChunks = 64; };  // 512 x 2 B

template <int FMT, int ST>
struct StreamShape {
    static constexpr int kChunks = StreamFmt<FMT>::kChunks;   // chunks per full row slice
    static constexpr int kLoads = (ST * kChunks + 63) / 64;   // loads per lane per tile
    static constexpr int kBufBytes = kLoads * 64 * 16;        // per-wave LDS buffer
};

template <int FMT>
__device__ __forceinline__ typename Fmt<FMT>::Raw lds_lane(const uint8_t* row_slice, int li) {
    using F = Fmt<FMT>;
    typename F::Raw r;
    if constexpr (FMT == QG_FMT_Q8_0) {
        const uint8_t* blk = row_slice + (li >> 1) * 34;
        const U4u q = *reinterpret_cast<const U4u*>(blk + 2 + 16 * (li & 1));
        r.c[0] = q.v[0]; r.c[1] = q.v[1]; r.c[2] = q.v[2]; r.c[3] = q.v[3];
        r.d = *reinterpret_cast<const uint16_t*>(blk);
    } else if constexpr (FMT == QG_FMT_Q4_0) {
        const uint8_t* blk = row_slice + (li >> 1) * 18;
        const U2u q = *reinterpret_cast<const U2u*>(blk + 2 + 8 * (li & 1));
        r.c[0] = q.v[0]; r.c[1] = q.v[1];
        r.d = *reinterpret_cast<const uint16_t*>(blk);
    } else {
        const U4a* p = reinterpret_cast<const U4a*>(row_slice + 32 * li);
        const U4a a = p[0], b = p[1];
        r.c[0] = a.v[0]; r.c[1] = a.v[1]; r.c[2] = a.v[2]; r.c[3] = a.v[3];
        r.c[4] = b.v[0]; r.c[5] = b.v[1]; r.c[6] = b.v[2]; r.c[7] = b.v[3];
    }
    return r;
}

// Buffer-resource word 3 for gfx9-family (CDNA) raw buffer loads.
constexpr int kBufferRsrcWord3 = 0x00020000;
// Byte offset no tile reaches: a lane loading from it gets zeros, no memory access.
constexpr int kNoLoad = 0x7FFFFFF0;

// Tile t of the workgroup's rows, one 16-byte chunk per lane per load, through a
// buffer descriptor that covers exactly the tile's rows: padding lanes (offset
// kNoLoad) and rows past the end fall outside it and are skipped by the
// hardware; a tile past the last gets an empty descriptor.  Every load is
// issued unconditionally, so wait counts stay exact.
template <int FMT, int ST>
__device__ __forceinline__ void stream_issue(const uint8_t* __restrict__ W, int64_t row_bytes, int64_t row_begin,
                                             int64_t row_end, int ntiles, int t,
                                             const int (&off)[StreamShape<FMT, ST>::kLoads],
                                             V4 (&R)[StreamShape<FMT, ST>::kLoads]) {
    constexpr int L = StreamShape<FMT, ST>::kLoads;
    const bool live = t < ntiles;
    const int64_t r0 = row_begin + (int64_t)(live ? t : 0) * ST;
    const int64_t rows_here = row_end - r0 < ST ? row_end - r0 : ST;
    const int num = live ? (int)(rows_here * row_bytes) : 0;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(W + r0 * row_bytes), (short)0, num, kBufferRsrcWord3);
#pragma unroll
    for (int k = 0; k < L; ++k) R[k] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off[k], 0, 0);
}

// Decode, multiply and reduce one tile that sits in the wave's LDS buffer (chunk
// order), and write the wave's partial sums for it.
template <int FMT, int NT, int ST>
__device__ __forceinline__ void tile_compute(const uint8_t* buf, float* part, const float (&xr)[NT][kWeightsPerLane],
                                             int li, int g, int s, int nsl, int t, bool lane_ok, bool upper_ok,
                                             int my_idx, bool writer) {
    using F = Fmt<FMT>;
    using S = StreamShape<FMT, ST>;
    constexpr int TP = pad_pow2(NT);
    constexpr int RB = ST / 2;
    constexpr int N = RB * TP;
    typename F::Raw raw[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) raw[i] = lds_lane<FMT>(buf + (2 * i + g) * (S::kChunks * 16), li);
    float acc[RB][TP];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int n = 0; n < TP; ++n) acc[i][n] = 0.0f;
    accumulate_batch<FMT, NT, RB>(raw, xr, lane_ok, upper_ok, acc);
    float v[N];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int n = 0; n < TP; ++n) v[i * TP + n] = acc[i][n];
    butterfly32<N>(v, li);
    if (writer) part[(((size_t)t * nsl + s) * 2 + g) * N + my_idx] = v[0];
}

template <int FMT, int NT, int ST>
__device__ __forceinline__ void stream_tile(const uint8_t* __restrict__ W, int64_t row_bytes, int64_t row_begin,
                                            int64_t row_end, int ntiles, int t, int ahead,
                                            const int (&off)[StreamShape<FMT, ST>::kLoads],
                                            V4 (&R)[StreamShape<FMT, ST>::kLoads], uint8_t* buf, float* part,
                                            const float (&xr)[NT][kWeightsPerLane], int lane, int li, int g, int s,
                                            int nsl, bool lane_ok, bool upper_ok, int my_idx, bool writer) {
    constexpr int L = StreamShape<FMT, ST>::kLoads;
    // registers -> LDS (chunk order), then the next-but-one tile into R
#pragma unroll
    for (int k = 0; k < L; ++k) *reinterpret_cast<V4*>(buf + (64 * k + lane) * 16) = R[k];
    stream_issue<FMT, ST>(W, row_bytes, row_begin, row_end, ntiles, t + ahead, off, R);
    tile_compute<FMT, NT, ST>(buf, part, xr, li, g, s, nsl, t, lane_ok, upper_ok, my_idx, writer);
}

template <int FMT, int NT, int ST, class Out>
__device__ __forceinline__ void stream_rows(const uint8_t* __restrict__ W, int64_t row_bytes, int cols, int nsl,
                                            const float* __restrict__ x, const int64_t (&xoff)[NT], int64_t row_begin,
                                            int64_t row_end, int nw, Out&& out) {
    using F = Fmt<FMT>;
    using S = StreamShape<FMT, ST>;
    constexpr int TP = pad_pow2(NT);
    constexpr int RB = ST / 2;      // rows per 32-lane group per tile
    constexpr int N = RB * TP;      // values per lane entering the butterfly
    constexpr int L = S::kLoads;
    static_assert(N <= 32, "tile rows * tokens too large");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps buffer descriptors scalar
    // nw: waves per workgroup, an argument
    const int g = lane >> 5;
    const int li = lane & 31;
    // waves = slices x row groups: wave (s, rg) takes k slice s of tiles rg, rg + RG, ...
    const int s = wave % nsl;
    const int rg = wave / nsl;
    const int RG = nw / nsl;
    const int k0 = s * kSlice;
    const int ntiles = (int)((row_end - row_begin + ST - 1) / ST);
    uint8_t* buf = smem + wave * S::kBufBytes;
    float* part = reinterpret_cast<float*>(smem + nw * S::kBufBytes);  // [tiles, rounded up to 2*RG][nsl][2][N]

    // chunks of this wave's slice that exist (the last slice of a row may be short)
    const int64_t rest = row_bytes - (int64_t)s * S::kChunks * 16;
    const int cs = rest / 16 < S::kChunks ? (int)(rest / 16) : S::kChunks;
    // lane's chunk of load k: byte offset inside the tile (the same for every tile)
    int off[L];
#pragma unroll
    for (int k = 0; k < L; ++k) {
        const int j = 64 * k + lane;
        const int r = j / S::kChunks, c = j % S::kChunks;
        off[k] = (r < ST && c < cs) ? (int)(r * row_bytes) + s * S::kChunks * 16 + 16 * c : kNoLoad;
    }

    const bool lane_ok = F::lane_valid(li, k0, cols);
    const bool upper_ok = lane_ok && F::upper_valid(li, k0, cols);
    bool writer;
    const int my_idx = butterfly_index<N>(li, writer);
    float xr[NT][kWeightsPerLane];

    V4 ra[L], rb[L];
    load_x<FMT, NT>(x, xoff, k0, li, lane_ok, cols, xr);  // oldest loads first: waits inside the loop stay tight
    stream_issue<FMT, ST>(W, row_bytes, row_begin, row_end, ntiles, rg, off, ra);
    stream_issue<FMT, ST>(W, row_bytes, row_begin, row_end, ntiles, rg + RG, off, rb);
    for (int t = rg; t < ntiles; t += 2 * RG) {
        // both halves always run (a tile past the end loads nothing and its partial
        // slots are never read), so every iteration has the same wait pattern
        stream_tile<FMT, NT, ST>(W, row_bytes, row_begin, row_end, ntiles, t, 2 * RG, off, ra, buf, part, xr, lane, li,
                                 g, s, nsl, lane_ok, upper_ok, my_idx, writer);
        stream_tile<FMT, NT, ST>(W, row_bytes, row_begin, row_end, ntiles, t + RG, 2 * RG, off, rb, buf, part, xr, lane,
                                 li, g, s, nsl, lane_ok, upper_ok, my_idx, writer);
    }
    __syncthreads();
    // every output of the workgroup: sum the slices' partials in slice order
    const int nrows = (int)(row_end - row_begin);
    for (int o = tid; o < nrows * NT; o += blockDim.x) {
        const int rr = o / NT, t = o % NT;
        const int tl = rr / ST, rin = rr % ST;
        const int gg = rin & 1, i = rin >> 1;
        const float* base = part + ((size_t)tl * nsl * 2 + gg) * N + i * TP + t;
        float sum = base[0];
        for (int w = 1; w < nsl; ++w) sum = sum + base[(size_t)w * 2 * N];
        out(t, row_begin + rr, sum);
    }
}

// ------------------------------------------------- LDS-DMA streamed variant
// The same tiles and arithmetic as stream_rows, but the loads go straight into
// LDS (buffer_load ... lds: one 1 KB row of the wave's buffer per instruction,
// lane l's 16 bytes at offset 16 l, out-of-range lanes write zeros).  No
// registers hold tiles in flight, so a wave keeps D tiles in flight in a ring of
// D LDS slots -- for small matrices all of its tiles at once.
//
// The compiler does not order these loads against LDS reads, so the waits are
// explicit.  x comes in the same way (into the last slots of the ring, read into
// registers once, after which those slots take tiles), so no load of the kernel
// writes registers and the compiler adds no vmcnt waits of its own.  The wave
// always has exactly D tiles issued after the start (tiles past its last get an
// empty descriptor: every lane out of range), so before tile i is read at most
// (D - 1) * L newer loads may be outstanding; a slot is refilled only after its
// reads have returned (lgkmcnt(0)); all loads are drained before the workgroup
// ends, since an empty load still writes its zeros.
typedef __attribute__((address_space(3))) void lds_void_t;

// Cache policy of a load.  kStreamPolicy sets the non-temporal bit, so the caches
// keep the lines as streaming data that they give up first.  kSplitPolicy is a tag
// for the weight streams: a wave's row piece rarely starts or ends on a 128-byte
// line, so the lines at its two ends are shared with the neighbouring pieces, which
// other waves load; those chunks keep the default policy, so that the line stays
// for its second reader, and every other chunk streams (the bits are the same
// under any policy).  Measured per kernel kind: the persistent kind splits for Q8_0
// (the LM head: 225-230 µs at T = 1..4 with the default policy, 214-220 streaming,
// 203-210 split) and streams otherwise (kPersistPolicy); the dense matrix-core kinds
// stream for Q4_0 and BF16 only (kDensePolicy);
// the grouped experts, whose experts several tokens share, and the gathered row
// subset keep the default (streaming cost them 0.4-0.6 and 0.3-0.7 µs).
constexpr int kDefaultPolicy = 0;
constexpr int kStreamPolicy = 2;
constexpr int kSplitPolicy = -1;

// One direct-to-LDS load (16 bytes per lane).  The builtin only exists for the
// device; the host pass compiles an empty body it never runs.
template <int POLICY = kDefaultPolicy>
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, uint8_t* lds, int voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds, 16, voffset, 0, 0, POLICY);
#else
    (void)rsrc, (void)lds, (void)voffset;
#endif
}

// Bit k set: the 16-byte chunk this lane fetches in load k of a tile lies in a
// 128-byte line that also holds bytes of another row piece.  Lane l of load k
// fetches chunk 64 k + l of the tile, `chunks` chunks per row piece; the first row
// piece of the tile starts at byte `first` (an address: the line grid is absolute)
// and row r's at first + r * row_bytes.  The same for every tile of a range whose
// tiles lie a multiple of 128 bytes apart.
template <int LOADS>
__device__ __forceinline__ uint32_t shared_line_mask(uint64_t first, int64_t row_bytes, int chunks, int rows,
                                                     int lane) {
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
        const int j = 64 * k + lane;
        const int r = j / chunks, c = j % chunks;
        const uint64_t ps = first + (uint64_t)r * (uint64_t)row_bytes;  // the piece
        const uint64_t pe = ps + 16 * (uint64_t)chunks - 1;            // its last byte
        const uint64_t line = (ps + 16 * (uint64_t)c) >> 7;
        const bool head = (ps & 127) != 0 && line == (ps >> 7);
        const bool tail = ((pe + 1) & 127) != 0 && line == (pe >> 7);
        if (r < rows && (head || tail)) m |= 1u << k;
    }
    return m;
}

// One load of a weight stream under POLICY (kSplitPolicy: the default policy if
// `shared`, else streaming; the lanes of one load split into two masked loads).
template <int POLICY>
__device__ __forceinline__ void load_w16(__amdgpu_buffer_rsrc_t rsrc, uint8_t* lds, int voffset, bool shared) {
    if constexpr (POLICY == kSplitPolicy) {
        if (shared) load_lds16<kDefaultPolicy>(rsrc, lds, voffset);
        else load_lds16<kStreamPolicy>(rsrc, lds, voffset);
    } else {
        (void)shared;
        load_lds16<POLICY>(rsrc, lds, voffset);
    }
}

// q = a / b, r = a % b for 0 <= a < 16 and b >= 1 (the waves and slices of a
// workgroup): a short scalar loop in place of a general 32-bit division, which
// sits in front of a wave's first load (measured 0.03-0.1 µs per call on the
// 2560-column mat-vecs).
__device__ __forceinline__ void small_divmod(int a, int b, int& q, int& r) {
    q = 0;
    r = a;
    if (b <= 0) return;  // never launched so (the host rejects cols <= 0); no endless loop either way
    while (r >= b) { r -= b; ++q; }
}

template <int V>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(V >= 0 && V <= 63, "vmcnt is 6 bits");
    // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
    __builtin_amdgcn_s_waitcnt((V & 15) | (7 << 4) | (15 << 8) | ((V >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14)); }


template <int FMT, int ST>
__device__ __forceinline__ void dma_issue(const uint8_t* __restrict__ W, int64_t row_bytes, int64_t row_begin,
                                          int64_t row_end, int ntiles, int t, const int (&off)[StreamShape<FMT, ST>::kLoads],
                                          uint8_t* lbuf) {
    constexpr int L = StreamShape<FMT, ST>::kLoads;
    const bool live = t < ntiles;
    const int64_t r0 = row_begin + (int64_t)(live ? t : 0) * ST;
    const int64_t rows_here = row_end - r0 < ST ? row_end - r0 : ST;
    const int num = live ? (int)(rows_here * row_bytes) : 0;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(W + r0 * row_bytes), (short)0, num, kBufferRsrcWord3);
#pragma unroll
    for (int k = 0; k < L; ++k)
        load_lds16(rsrc, lbuf + 1024 * k, off[k]);
}

// Slots of the ring that x[NT][512 of the slice] occupies at the start.
template <int FMT, int ST, int NT>
constexpr int dma_x_slots() { return (NT * kSlice * 4 + StreamShape<FMT, ST>::kBufBytes - 1) / StreamShape<FMT, ST>::kBufBytes; }

// XSEP: x gets a region of its own after the rings ([waves][NT][2 KB]), so all D
// tiles are issued at once; otherwise x borrows the last ring slots and the
// tiles for them are issued after x is read.
// Per-lane byte offsets of a wave's loads within a tile of its slice s.
template <int FMT, int ST>
__device__ __forceinline__ void tile_offsets(int64_t row_bytes, int s, int lane, int (&off)[StreamShape<FMT, ST>::kLoads]) {
    using S = StreamShape<FMT, ST>;
    const int64_t rest = row_bytes - (int64_t)s * S::kChunks * 16;
    const int cs = rest / 16 < S::kChunks ? (int)(rest / 16) : S::kChunks;
#pragma unroll
    for (int k = 0; k < S::kLoads; ++k) {
        const int j = 64 * k + lane;
        const int r = j / S::kChunks, c = j % S::kChunks;
        off[k] = (r < ST && c < cs) ? (int)(r * row_bytes) + s * S::kChunks * 16 + 16 * c : kNoLoad;
    }
}

// The first D tiles of the wave's ring, issued before x is known (dma_rows with
// PRE then skips them): lets a caller start the weight stream while it still
// works out which activations apply.
template <int FMT, int ST, int D>
__device__ __forceinline__ void dma_prefetch(const uint8_t* __restrict__ W, int64_t row_bytes, int nsl, int64_t row_begin,
                                             int64_t row_end) {
    using S = StreamShape<FMT, ST>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int s = wave % nsl, rg = wave / nsl, RG = nw / nsl;
    const int ntiles = (int)((row_end - row_begin + ST - 1) / ST);
    int off[S::kLoads];
    tile_offsets<FMT, ST>(row_bytes, s, lane, off);
#pragma unroll
    for (int i = 0; i < D; ++i)
        dma_issue<FMT, ST>(W, row_bytes, row_begin, row_end, ntiles, rg + i * RG, off,
                           smem + (wave * D + i) * S::kBufBytes);
}

template <int FMT, int NT, int ST, int D, bool XSEP, class Out, bool PRE = false>
__device__ __forceinline__ void dma_rows(const uint8_t* __restrict__ W, int64_t row_bytes, int cols, int nsl,
                                         const float* __restrict__ x, const int64_t (&xoff)[NT], int64_t row_begin,
                                         int64_t row_end, int nw, Out&& out) {
    static_assert(!PRE || XSEP, "prefetched tiles need x staged apart");
    using F = Fmt<FMT>;
    using S = StreamShape<FMT, ST>;
    constexpr int TP = pad_pow2(NT);
    constexpr int RB = ST / 2;
    constexpr int N = RB * TP;
    constexpr int L = S::kLoads;
    constexpr int X = XSEP ? 0 : dma_x_slots<FMT, ST, NT>();
    static_assert(N <= 32, "tile rows * tokens too large");
    static_assert(X < D, "x must leave at least one slot for the first tile");
    static_assert((D - 1) * L <= 63, "vmcnt holds at most 63 outstanding loads");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps descriptors and M0 scalar
    // nw: waves per workgroup (an argument, so no load of the dispatch's sizes)
    const int g = lane >> 5;
    const int li = lane & 31;
    const int s = wave % nsl;
    const int rg = wave / nsl;
    const int RG = nw / nsl;
    const int k0 = s * kSlice;
    const int ntiles = (int)((row_end - row_begin + ST - 1) / ST);
    uint8_t* ring = smem + wave * D * S::kBufBytes;
    uint8_t* xl = XSEP ? smem + nw * D * S::kBufBytes + wave * NT * 2048 : ring + (D - X) * S::kBufBytes;
    float* part = reinterpret_cast<float*>(smem + nw * (D * S::kBufBytes + (XSEP ? NT * 2048 : 0)));  // [tiles][nsl][2][N]

    int off[L];
    tile_offsets<FMT, ST>(row_bytes, s, lane, off);
    const bool lane_ok = F::lane_valid(li, k0, cols);
    const bool upper_ok = lane_ok && F::upper_valid(li, k0, cols);
    bool writer;
    const int my_idx = butterfly_index<N>(li, writer);

    // x of the slice, token n at xl + 2048 n (k past cols reads as zero), then the
    // first D - X tiles (with PRE the D tiles are already on their way, older than x)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const __amdgpu_buffer_rsrc_t xr_rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)(x + xoff[n] + k0), (short)0, (cols - k0) * 4, kBufferRsrcWord3);
        load_lds16(xr_rsrc, xl + 2048 * n, 16 * lane);
        load_lds16(xr_rsrc, xl + 2048 * n + 1024, 16 * lane + 1024);
    }
    if constexpr (PRE) {
        wait_vmcnt<0>();  // x is the newest load
    } else {
#pragma unroll
        for (int i = 0; i < D - X; ++i)
            dma_issue<FMT, ST>(W, row_bytes, row_begin, row_end, ntiles, rg + i * RG, off, ring + i * S::kBufBytes);
        // x and tile 0 have landed once at most (D - X - 1) * L newer loads remain
        wait_vmcnt<(D - X - 1) * L>();
    }
    float xr[NT][kWeightsPerLane];
    {
        const int b0 = F::kbase(li, 0), b1 = F::kbase(li, 1);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const float4* p0 = reinterpret_cast<const float4*>(xl + 2048 * n + 4 * b0);
            const float4* p1 = reinterpret_cast<const float4*>(xl + 2048 * n + 4 * b1);
            const float4 a = p0[0], b = p0[1], c = p1[0], d = p1[1];
            xr[n][0] = a.x; xr[n][1] = a.y; xr[n][2] = a.z; xr[n][3] = a.w;
            xr[n][4] = b.x; xr[n][5] = b.y; xr[n][6] = b.z; xr[n][7] = b.w;
            xr[n][8] = c.x; xr[n][9] = c.y; xr[n][10] = c.z; xr[n][11] = c.w;
            xr[n][12] = d.x; xr[n][13] = d.y; xr[n][14] = d.z; xr[n][15] = d.w;
        }
    }
    if constexpr (X > 0) {
        wait_lgkmcnt0();  // x is in registers: its slots take tiles D - X .. D - 1
#pragma unroll
        for (int i = D - X; i < D; ++i)
            dma_issue<FMT, ST>(W, row_bytes, row_begin, row_end, ntiles, rg + i * RG, off, ring + i * S::kBufBytes);
    }

    // this wave's tiles: rg, rg + RG, ...
    const int mine = ntiles > rg ? (ntiles - rg + RG - 1) / RG : 0;
    for (int i = 0; i < mine; ++i) {
        uint8_t* buf = ring + (i % D) * S::kBufBytes;
        wait_vmcnt<(D - 1) * L>();
        tile_compute<FMT, NT, ST>(buf, part, xr, li, g, s, nsl, rg + i * RG, lane_ok, upper_ok, my_idx, writer);
        wait_lgkmcnt0();
        dma_issue<FMT, ST>(W, row_bytes, row_begin, row_end, ntiles, rg + (i + D) * RG, off, buf);
    }
    wait_vmcnt<0>();
    __syncthreads();
    // every output of the workgroup: sum the slices' partials in slice order
    const int nrows = (int)(row_end - row_begin);
    for (int o = tid; o < nrows * NT; o += blockDim.x) {
        const int rr = o / NT, t = o % NT;
        const int tl = rr / ST, rin = rr % ST;
        const int gg = rin & 1, i = rin >> 1;
        const float* base = part + ((size_t)tl * nsl * 2 + gg) * N + i * TP + t;
        float sum = base[0];
        for (int w = 1; w < nsl; ++w) sum = sum + base[(size_t)w * 2 * N];
        out(t, row_begin + rr, sum);
    }
}

// ------------------------------------------------ half slices: 16 lanes per row
// The LDS-DMA kernel with k cut into 256-wide slices (8 blocks: 272 / 144 bytes
// of a Q8_0 / Q4_0 row, 512 of a BF16 row) and one wave per slice: a 32-column-block matrix of 10240 x 2560 runs ten
// waves per workgroup, three or two per SIMD with half a slice's work each,
// instead of five waves that put two full shares on one SIMD.  A row's 16 lanes
// own 16 weights each (the lane layout of the 512-wide kernels, blocks 0..7);
// the four 16-lane groups of a wave take rows g and g + 4 of an 8-row tile, and
// reduce over their 16 lanes with the four DPP stages of the halving butterfly.
// Slices are summed in order at the end, so a token's bits do not depend on T.
constexpr int kHalfSlice = 256;
template <int FMT>
struct HalfShape {  // 8-row tiles
    static constexpr int kChunks = StreamFmt<FMT>::kChunks / 2;  // 16-byte chunks per row slice: 17, 9, 32
    static constexpr int kLoads = (8 * kChunks + 63) / 64;       // 3, 2, 4
    static constexpr int kBufBytes = kLoads * 1024;              // per ring slot
};

template <int N>
__device__ __forceinline__ void butterfly16(float (&v)[N], int li) {
    constexpr int ctrls[4] = {0x140, 0x141, 0x4E, 0xB1};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const int m = 8 >> st;
        const int cnt = N >> st;
        if (cnt >= 2) {
            const bool up = (li & m) != 0;
#pragma unroll
            for (int i = 0; i < cnt / 2; ++i) {
                const float lo = v[i] + dpp_f(v[i], ctrls[st]);
                const float hi = v[i + cnt / 2] + dpp_f(v[i + cnt / 2], ctrls[st]);
                v[i] = up ? hi : lo;
            }
        } else {
            v[0] = v[0] + dpp_f(v[0], ctrls[st]);
        }
    }
}

template <int N>
__device__ __forceinline__ int butterfly16_index(int li, bool& writer) {
    int idx = 0;
    writer = true;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const int m = 8 >> st;
        const int cnt = N >> st;
        if (cnt >= 2) {
            if (li & m) idx += cnt / 2;
        } else if (li & m) {
            writer = false;
        }
    }
    return idx;
}

// Lane l of load k fetches chunk j = 64 k + l of the tile's slice: row j / C,
// chunk j % C (past the tile's 8 rows or the slice's chunks: nothing, zeros).
template <int FMT>
__device__ __forceinline__ void half_offsets(int64_t row_bytes, int s, int lane, int (&off)[HalfShape<FMT>::kLoads]) {
    using H = HalfShape<FMT>;
    const int64_t rest = row_bytes - (int64_t)s * H::kChunks * 16;
    const int cs = rest / 16 < H::kChunks ? (int)(rest / 16) : H::kChunks;
#pragma unroll
    for (int k = 0; k < H::kLoads; ++k) {
        const int j = 64 * k + lane;
        const int r = j / H::kChunks, c = j % H::kChunks;
        off[k] = (r < 8 && c < cs) ? (int)(r * row_bytes) + s * H::kChunks * 16 + 16 * c : kNoLoad;
    }
}

template <int FMT>
__device__ __forceinline__ void half_issue(const uint8_t* __restrict__ W, int64_t row_bytes, int64_t row_begin,
                                           int64_t row_end, int ntiles, int t, const int (&off)[HalfShape<FMT>::kLoads],
                                           uint8_t* lbuf) {
    const bool live = t < ntiles;
    const int64_t r0 = row_begin + (int64_t)(live ? t : 0) * 8;
    const int64_t rows_here = row_end - r0 < 8 ? row_end - r0 : 8;
    const int num = live ? (int)(rows_here * row_bytes) : 0;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(W + r0 * row_bytes), (short)0, num, kBufferRsrcWord3);
#pragma unroll
    for (int k = 0; k < HalfShape<FMT>::kLoads; ++k) load_lds16(rsrc, lbuf + 1024 * k, off[k]);
}

template <int FMT, int NT, int D, class Out>
__device__ __forceinline__ void half_rows(const uint8_t* __restrict__ W, int64_t row_bytes, int cols, int nsl,
                                          const float* __restrict__ x, int64_t row_begin, int64_t row_end, int nw,
                                          Out&& out) {
    using F = Fmt<FMT>;
    using H = HalfShape<FMT>;
    constexpr int TP = pad_pow2(NT);
    constexpr int RB = 2;  // rows per 16-lane group per tile
    constexpr int N = RB * TP;
    constexpr int L = H::kLoads;
    static_assert(D * L <= 63, "vmcnt holds at most 63 outstanding loads");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps descriptors and M0 scalar
    const int g = lane >> 4;   // 16-lane group: rows g and g + 4 of a tile
    const int li = lane & 15;
    const int s = wave % nsl, rg = wave / nsl, RG = nw / nsl;
    const int k0 = s * kHalfSlice;
    const int ntiles = (int)((row_end - row_begin + 7) / 8);
    uint8_t* ring = smem + wave * D * H::kBufBytes;
    uint8_t* xl = smem + nw * D * H::kBufBytes + wave * NT * 1024;          // x[NT][256] of the slice
    float* part = reinterpret_cast<float*>(smem + nw * (D * H::kBufBytes + NT * 1024));  // [tiles][nsl][4][N]

    int off[L];
    half_offsets<FMT>(row_bytes, s, lane, off);
    const bool lane_ok = F::lane_valid(li, k0, cols);
    const bool upper_ok = lane_ok && F::upper_valid(li, k0, cols);
    bool writer;
    const int my_idx = butterfly16_index<N>(li, writer);

    // x of the slice (k past cols reads as zero), then the first D tiles
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const __amdgpu_buffer_rsrc_t xr_rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)(x + (int64_t)n * cols + k0), (short)0, (cols - k0) * 4,
                                              kBufferRsrcWord3);
        load_lds16(xr_rsrc, xl + 1024 * n, 16 * lane);
    }
#pragma unroll
    for (int i = 0; i < D; ++i)
        half_issue<FMT>(W, row_bytes, row_begin, row_end, ntiles, rg + i * RG, off, ring + i * H::kBufBytes);
    wait_vmcnt<D * L>();  // x is older than every tile
    float xr[NT][kWeightsPerLane];
    {
        const int b0 = F::kbase(li, 0), b1 = F::kbase(li, 1);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const float4* p0 = reinterpret_cast<const float4*>(xl + 1024 * n + 4 * b0);
            const float4* p1 = reinterpret_cast<const float4*>(xl + 1024 * n + 4 * b1);
            const float4 a = p0[0], b = p0[1], c = p1[0], d = p1[1];
            xr[n][0] = a.x; xr[n][1] = a.y; xr[n][2] = a.z; xr[n][3] = a.w;
            xr[n][4] = b.x; xr[n][5] = b.y; xr[n][6] = b.z; xr[n][7] = b.w;
            xr[n][8] = c.x; xr[n][9] = c.y; xr[n][10] = c.z; xr[n][11] = c.w;
            xr[n][12] = d.x; xr[n][13] = d.y; xr[n][14] = d.z; xr[n][15] = d.w;
        }
    }

    const int mine = ntiles > rg ? (ntiles - rg + RG - 1) / RG : 0;
    for (int i = 0; i < mine; ++i) {
        uint8_t* buf = ring + (i % D) * H::kBufBytes;
        const int t = rg + i * RG;
        wait_vmcnt<(D - 1) * L>();
        typename F::Raw raw[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) raw[r] = lds_lane<FMT>(buf + (4 * r + g) * (H::kChunks * 16), li);
        float acc[RB][TP];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int n = 0; n < TP; ++n) acc[r][n] = 0.0f;
        accumulate_batch<FMT, NT, RB>(raw, xr, lane_ok, upper_ok, acc);
        float v[N];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int n = 0; n < TP; ++n) v[r * TP + n] = acc[r][n];
        butterfly16<N>(v, li);
        if (writer) part[(((size_t)t * nsl + s) * 4 + g) * N + my_idx] = v[0];
        // the slot is refilled once its reads have returned; refilling it before the
        // math (as soon as the bytes are in registers) measured slower at T >= 2
        wait_lgkmcnt0();
        half_issue<FMT>(W, row_bytes, row_begin, row_end, ntiles, rg + (i + D) * RG, off, buf);
    }
    wait_vmcnt<0>();
    __syncthreads();
    // every output of the workgroup: sum the slices' partials in slice order
    const int nrows = (int)(row_end - row_begin);
    for (int o = tid; o < nrows * NT; o += blockDim.x) {
        const int rr = o / NT, tk = o % NT;
        const int tl = rr / 8, rin = rr % 8;
        const int gg = rin & 3, r = rin >> 2;
        const float* base = part + ((size_t)tl * nsl * 4 + gg) * N + r * TP + tk;
        float sum = base[0];
        for (int w = 1; w < nsl; ++w) sum = sum + base[(size_t)w * 4 * N];
        out(tk, row_begin + rr, sum);
    }
}

// ------------------------------------------------------ row-subset (gather)
// The mat-vec over a list of rows, y[t][i] = W[ids[i]] . x[t] (the draft-vocabulary
// LM head in the mlxcel drafter-cost issue: the drafter reads only the rows of the
// tokens it may propose).  As dma_rows (x in registers, loaded with the ids before
// any load to LDS, so the ring needs no slots for it), but a tile's 8 rows
// are ids[...] of the workgroup's range: every wave first loads those ids (two
// per lane, at most 128 per workgroup: id j sits in lane j % 64 of register
// j / 64), and each load lane takes its row's id from the lane that holds it.  The descriptor spans all of W (< 2 GB, so every
// byte offset fits the 32-bit offset); an id outside [0, rows) loads nothing and
// its outputs are NaN.
template <int FMT, int NT, int D, class Out>
__device__ __forceinline__ void gather_rows(const uint8_t* __restrict__ W, int64_t rows, int64_t row_bytes, int cols,
                                            int nsl, const int32_t* __restrict__ ids, const float* __restrict__ x,
                                            int64_t sel_begin, int64_t sel_end, Out&& out) {
    using F = Fmt<FMT>;
    constexpr int ST = 8;
    using S = StreamShape<FMT, ST>;
    constexpr int TP = pad_pow2(NT);
    constexpr int RB = ST / 2;
    constexpr int N = RB * TP;
    constexpr int L = S::kLoads;
    static_assert((D - 1) * L <= 63, "vmcnt holds at most 63 outstanding loads");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = blockDim.x >> 6;
    const int g = lane >> 5, li = lane & 31;
    const int s = wave % nsl, rg = wave / nsl, RG = nw / nsl;
    const int k0 = s * kSlice;
    const int nsel = (int)(sel_end - sel_begin);  // <= 128
    const int ntiles = (nsel + ST - 1) / ST;
    uint8_t* ring = smem + wave * D * S::kBufBytes;
    float* part = reinterpret_cast<float*>(smem + nw * D * S::kBufBytes);  // [tiles][nsl][2][N]

    // the workgroup's row ids (two per lane) and the slice of x, into registers,
    // all complete before the first load to LDS
    const int my_id0 = lane < nsel ? ids[sel_begin + lane] : -1;
    const int my_id1 = 64 + lane < nsel ? ids[sel_begin + 64 + lane] : -1;
    const int64_t rest = row_bytes - (int64_t)s * S::kChunks * 16;
    const int cs = rest / 16 < S::kChunks ? (int)(rest / 16) : S::kChunks;
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void*)W, (short)0, (int)(rows * row_bytes), kBufferRsrcWord3);
    auto issue = [&](int t, uint8_t* lbuf) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < L; ++k) {
            const int j = 64 * k + lane;
            const int r = j / S::kChunks, c = j % S::kChunks;
            const int src = t * ST + r;  // the row's place in the range; tile t < 8 reads ids 0..63
            const int id = __shfl(t < 64 / ST ? my_id0 : my_id1, src & 63, 64);
            const bool live = t < ntiles && r < ST && src < nsel && c < cs && id >= 0 && id < rows;
            load_lds16(wr, lbuf + 1024 * k, live ? (int)(id * row_bytes) + s * S::kChunks * 16 + 16 * c : kNoLoad);
        }
    };

    const bool lane_ok = F::lane_valid(li, k0, cols);
    const bool upper_ok = lane_ok && F::upper_valid(li, k0, cols);
    bool writer;
    const int my_idx = butterfly_index<N>(li, writer);
    int64_t xoff[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) xoff[n] = (int64_t)n * cols;
    float xr[NT][kWeightsPerLane];
    load_x<FMT, NT>(x, xoff, k0, li, lane_ok, cols, xr);
    wait_vmcnt<0>();  // ids and x are in registers
#pragma unroll
    for (int i = 0; i < D; ++i) issue(rg + i * RG, ring + i * S::kBufBytes);
    const int mine = ntiles > rg ? (ntiles - rg + RG - 1) / RG : 0;
    for (int i = 0; i < mine; ++i) {
        uint8_t* buf = ring + (i % D) * S::kBufBytes;
        wait_vmcnt<(D - 1) * L>();
        tile_compute<FMT, NT, ST>(buf, part, xr, li, g, s, nsl, rg + i * RG, lane_ok, upper_ok, my_idx, writer);
        wait_lgkmcnt0();
        issue(rg + (i + D) * RG, buf);
    }
    wait_vmcnt<0>();
    __syncthreads();
    for (int o = tid; o < nsel * NT; o += blockDim.x) {
        const int rr = o / NT, t = o % NT;
        const int tl = rr / ST, rin = rr % ST;
        const int gg = rin & 1, i = rin >> 1;
        const float* base = part + ((size_t)tl * nsl * 2 + gg) * N + i * TP + t;
        float sum = base[0];
        for (int w = 1; w < nsl; ++w) sum = sum + base[(size_t)w * 2 * N];
        const int id = ids[sel_begin + rr];
        out(t, sel_begin + rr, id >= 0 && id < rows ? sum : __builtin_nanf(""));
    }
}

// ------------------------------------------------- unit-balanced DMA variant
// Work units are (k slice, 8-row tile) pairs of the workgroup's rows, in
// slice-major order; wave w of NW takes the contiguous range
// [w U / NW, (w + 1) U / NW) of the U units, so every wave (and every SIMD) gets
// the same work to within one unit whatever the number of slices.  The whole of
// x[T][cols] is staged in LDS once per workgroup (each wave loads a share, then
// one barrier); a wave reloads its x registers from LDS when its slice changes.
// Units stream through a ring of D LDS slots with the waits of dma_rows.  Each
// unit's arithmetic and the final slice-order sum are those of the other
// kinds, so the results are bit for bit the same.
template <int FMT, int NT, int D, class Out>
__device__ __forceinline__ void unit_rows(const uint8_t* __restrict__ W, int64_t row_bytes, int cols, int nsl,
                                          const float* __restrict__ x, int64_t row_begin, int64_t row_end, Out out) {
    using F = Fmt<FMT>;
    constexpr int ST = 8;
    using S = StreamShape<FMT, ST>;
    constexpr int TP = pad_pow2(NT);
    constexpr int RB = ST / 2;
    constexpr int N = RB * TP;
    constexpr int L = S::kLoads;
    static_assert(D * L <= 63, "vmcnt holds at most 63 outstanding loads");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = blockDim.x >> 6;
    const int g = lane >> 5;
    const int li = lane & 31;
    const int ntiles = (int)((row_end - row_begin + ST - 1) / ST);
    const int xbytes = NT * cols * 4;
    uint8_t* xl = smem;                                                     // x[NT][cols]
    uint8_t* ring = smem + ((xbytes + 1023) & ~1023) + wave * D * S::kBufBytes;
    float* part = reinterpret_cast<float*>(smem + ((xbytes + 1023) & ~1023) + nw * D * S::kBufBytes);  // [tiles][nsl][2][N]

    // this wave's units
    const int U = nsl * ntiles;
    const int u0 = (int)((int64_t)wave * U / nw), u1 = (int)((int64_t)(wave + 1) * U / nw);

    // per-lane chunk geometry of one tile (row r, chunk c) for each load; the
    // slice only shifts the offset and bounds the chunks
    int rc_off[L], rc_c[L];
#pragma unroll
    for (int k = 0; k < L; ++k) {
        const int j = 64 * k + lane;
        const int r = j / S::kChunks, c = j % S::kChunks;
        rc_off[k] = r < ST ? (int)(r * row_bytes) + 16 * c : -1;
        rc_c[k] = c;
    }
    auto issue = [&](int u, uint8_t* lbuf) __attribute__((always_inline)) {
        const bool live = u < u1;
        const int su = live ? u / ntiles : 0, tu = live ? u % ntiles : ntiles;
        int off[L];
        const int64_t rest = row_bytes - (int64_t)su * S::kChunks * 16;
        const int cs = rest / 16 < S::kChunks ? (int)(rest / 16) : S::kChunks;
#pragma unroll
        for (int k = 0; k < L; ++k)
            off[k] = (rc_off[k] >= 0 && rc_c[k] < cs) ? rc_off[k] + su * S::kChunks * 16 : kNoLoad;
        dma_issue<FMT, ST>(W, row_bytes, row_begin, row_end, ntiles, tu, off, lbuf);
    };

    // x: 1 KB pieces of the flattened x[NT][cols], shared out round-robin
    {
        const __amdgpu_buffer_rsrc_t xr_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, xbytes, kBufferRsrcWord3);
        const int npieces = (xbytes + 1023) / 1024;
        for (int j = wave; j < npieces; j += nw) load_lds16(xr_rsrc, xl + 1024 * j, 1024 * j + 16 * lane);
    }
#pragma unroll
    for (int i = 0; i < D; ++i) issue(u0 + i, ring + i * S::kBufBytes);
    wait_vmcnt<D * L>();  // this wave's share of x has landed ...
    // ... and every other wave's.  A bare s_barrier: __syncthreads() would also
    // wait for the tiles in flight.  The empty asm keeps the compiler from moving
    // LDS accesses across it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    float xr[NT][kWeightsPerLane];
    int cur = -1;
    bool lane_ok = false, upper_ok = false;
    bool writer;
    const int my_idx = butterfly_index<N>(li, writer);
    for (int u = u0; u < u1; ++u) {
        const int i = u - u0;
        const int su = u / ntiles, tu = u % ntiles;
        if (su != cur) {  // uniform
            cur = su;
            const int k0 = su * kSlice;
            lane_ok = F::lane_valid(li, k0, cols);
            upper_ok = lane_ok && F::upper_valid(li, k0, cols);
            // x of the slice (a lane past cols reads its token's first values; its
            // products are discarded)
            const int b0 = lane_ok ? k0 + F::kbase(li, 0) : 0;
            const int b1 = lane_ok ? k0 + F::kbase(li, 1) : 0;
            const int b1c = b1 + 8 <= cols ? b1 : b0;
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const float4* p0 = reinterpret_cast<const float4*>(xl + 4 * (n * cols + b0));
                const float4* p1 = reinterpret_cast<const float4*>(xl + 4 * (n * cols + b1c));
                const float4 a = p0[0], b = p0[1], c = p1[0], d = p1[1];
                xr[n][0] = a.x; xr[n][1] = a.y; xr[n][2] = a.z; xr[n][3] = a.w;
                xr[n][4] = b.x; xr[n][5] = b.y; xr[n][6] = b.z; xr[n][7] = b.w;
                xr[n][8] = c.x; xr[n][9] = c.y; xr[n][10] = c.z; xr[n][11] = c.w;
                xr[n][12] = d.x; xr[n][13] = d.y; xr[n][14] = d.z; xr[n][15] = d.w;
            }
        }
        uint8_t* buf = ring + (i % D) * S::kBufBytes;
        wait_vmcnt<(D - 1) * L>();
        tile_compute<FMT, NT, ST>(buf, part, xr, li, g, su, nsl, tu, lane_ok, upper_ok, my_idx, writer);
        wait_lgkmcnt0();
        issue(u + D, buf);
    }
    wait_vmcnt<0>();
    __syncthreads();
    const int nrows = (int)(row_end - row_begin);
    for (int o = tid; o < nrows * NT; o += blockDim.x) {
        const int rr = o / NT, t = o % NT;
        const int tl = rr / ST, rin = rr % ST;
        const int gg = rin & 1, i = rin >> 1;
        const float* base = part + ((size_t)tl * nsl * 2 + gg) * N + i * TP + t;
        float sum = base[0];
        for (int w = 1; w < nsl; ++w) sum = sum + base[(size_t)w * 2 * N];
        out(t, row_begin + rr, sum);
    }
}

// ------------------------------------------------------ matrix-core variant
// The same streamed tiles (16 rows), contracted on the matrix cores with
// v_mfma_f32_16x16x32_bf16: D[16 x 16] = A[16 x 32] . B[32 x 16] per block.
//   A: activations.  Row m = 4p + t holds piece p (< 3) of token t (< 4); every
//      fp32 x is split exactly into three bf16 pieces, x = hi + mid + lo (each
//      residual is exact in fp32 and fits 8 significant bits by the third).
//   B: one block of 16 weight rows; column n = weight row, the 32 codes as bf16
//      (exact: |code| <= 128).
//   Products are exact in fp32; per block, lane l gets D rows 4(l/16)..+3 of
//   column l%16 -- one weight row, so one scale: acc += d * D.  At the end the
//   three pieces of a token are added in a fixed order.  A token's outputs never
//   depend on the other tokens' rows of A, so its bits do not depend on T.
typedef __bf16 BF8 __attribute__((ext_vector_type(8)));
typedef float F4 __attribute__((ext_vector_type(4)));

// 8 int8 codes (two dwords) -> 8 bf16 (the high half of each exact fp32)
__device__ __forceinline__ V4 codes_to_bf16(uint32_t c0, uint32_t c1) {
    V4 r;
    const uint32_t w[2] = {c0, c1};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t f0 = __builtin_bit_cast(uint32_t, (float)(int32_t)(int8_t)(w[h]));
        const uint32_t f1 = __builtin_bit_cast(uint32_t, (float)(int32_t)(int8_t)(w[h] >> 8));
        const uint32_t f2 = __builtin_bit_cast(uint32_t, (float)(int32_t)(int8_t)(w[h] >> 16));
        const uint32_t f3 = __builtin_bit_cast(uint32_t, (float)(int32_t)(int8_t)(w[h] >> 24));
        r[2 * h] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);      // (hi16(f1) << 16) | hi16(f0)
        r[2 * h + 1] = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
    }
    return r;
}

// Piece p of x (bf16 bits) in an exact three-way split by truncation:
// hi = x with its low 16 bits cleared, mid = the same of x - hi, lo = x - hi - mid.
// x has a 24-bit significand: x - hi is exact and holds at most 16 significant
// bits, x - hi - mid at most 8, so lo is exactly a bf16 and hi + mid + lo = x.
// m1 = (p >= 1), m2 = (p >= 2) as 0/1 floats select the piece without branches:
// fma(-0, t, v) = v and fma(-1, t, v) = v - t, both exact.
__device__ __forceinline__ uint32_t x_piece(float x, float m1, float m2) {
    const float t1 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x) & 0xFFFF0000u);
    const float v1 = __builtin_fmaf(-m1, t1, x);
    const float t2 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v1) & 0xFFFF0000u);
    const float v2 = __builtin_fmaf(-m2, t2, v1);
    return __builtin_bit_cast(uint32_t, v2) >> 16;  // exact: v2's low 16 bits are zero when p == 2
}

// Loads of one 16-row Q8_0 tile (as stream_issue).  The per-lane byte offsets are
// recomputed at every issue from an opaque copy of the lane id, so they hold no
// registers across the loop (the A fragments need them).  j / 34 is exact as
// (j * 1928) >> 16 for every chunk index j < 578.
__device__ __forceinline__ void mfma_issue(const uint8_t* __restrict__ W, int row_bytes, int64_t row_begin,
                                           int64_t row_end, int ntiles, int t, int lane, int cs, int sbase,
                                           V4 (&R)[StreamShape<QG_FMT_Q8_0, 16>::kLoads]) {
    constexpr int L = StreamShape<QG_FMT_Q8_0, 16>::kLoads;
    static_assert(64 * L <= 578, "chunk index past the exact range of the division");
    int l = lane;
    asm volatile("" : "+v"(l));
    const bool live = t < ntiles;
    const int64_t r0 = row_begin + (int64_t)(live ? t : 0) * 16;
    const int64_t rows_here = row_end - r0 < 16 ? row_end - r0 : 16;
    const int num = live ? (int)(rows_here * row_bytes) : 0;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(W + r0 * row_bytes), (short)0, num, kBufferRsrcWord3);
#pragma unroll
    for (int k = 0; k < L; ++k) {
        const int j = 64 * k + l;
        const int r = (j * 1928) >> 16, c = j - 34 * r;
        const int o = (r < 16 && c < cs) ? r * row_bytes + sbase + 16 * c : kNoLoad;
        R[k] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, o, 0, 0);
    }
}

constexpr int kMfmaRowStride = 560;  // 16 rows x 560 B = 8960 B: within the 9 KB per-wave buffer
static_assert(16 * kMfmaRowStride <= StreamShape<QG_FMT_Q8_0, 16>::kBufBytes, "padded tile exceeds the wave buffer");

template <int NT>
__device__ __forceinline__ void mfma_tile_q8(const uint8_t* __restrict__ W, int row_bytes, int64_t row_begin,
                                             int64_t row_end, int ntiles, int t, int ahead, int cs, int sbase,
                                             V4 (&R)[StreamShape<QG_FMT_Q8_0, 16>::kLoads], uint8_t* buf, float* part,
                                             const V4 (&afrag)[16], int lane, int n, int g, int s, int nsl, int nblk,
                                             int pt) {
    using S = StreamShape<QG_FMT_Q8_0, 16>;
    constexpr int L = S::kLoads;
    constexpr int TP = pad_pow2(NT);
    // registers -> LDS with each 544-byte row slice at a 560-byte stride: the
    // 16 rows the B fragments read at once then fall in distinct banks
#pragma unroll
    for (int k = 0; k < L; ++k) {
        const int j = 64 * k + lane;
        const int r = (j * 1928) >> 16, c = j - 34 * r;  // j / 34, j % 34 (exact for j < 578)
        if (r < 16) *reinterpret_cast<V4*>(buf + r * kMfmaRowStride + 16 * c) = R[k];
    }
    mfma_issue(W, row_bytes, row_begin, row_end, ntiles, t + ahead, lane, cs, sbase, R);
    const uint8_t* rowp = buf + n * kMfmaRowStride;
    // Four accumulators (block b goes to b % 4) so consecutive blocks' matrix
    // products and scalings overlap; combined in a fixed order at the end.
    // Blocks past a short last slice read stale (finite) codes against zero A
    // fragments; their scale is forced to 0 so a stale Inf/NaN cannot leak in.
    // Only the first NJ of a lane's four rows of D carry tokens (A's rows of tokens
    // >= NT are zero): the scalings and the piece sums skip the rest.
    constexpr int NJ = NT < 4 ? NT : 4;
    F4 acc4[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) acc4[a] = F4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int b = 0; b < 16; ++b) {
        const uint8_t* blk = rowp + 34 * b;
        const U2u q = *reinterpret_cast<const U2u*>(blk + 2 + 8 * g);
        const float dv = half_bits_to_float(*reinterpret_cast<const uint16_t*>(blk));
        const float d = b < nblk ? dv : 0.0f;
        const V4 bq = codes_to_bf16(q.v[0], q.v[1]);
        const F4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        const F4 dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(BF8, afrag[b]),
                                                               __builtin_bit_cast(BF8, bq), z, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc4[b & 3][j] = __builtin_fmaf(d, dd[j], acc4[b & 3][j]);
    }
    F4 acc;
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = (acc4[0][j] + acc4[1][j]) + (acc4[2][j] + acc4[3][j]);
    // pieces of token j sit in lanes n (hi), n + 16 (mid), n + 32 (lo): added in
    // that order.  permlane16_swap brings lane n + 16's value to lane n (rows 0/1
    // of the wave trade places), permlane32_swap lane n + 32's (halves trade).
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        float mid = acc[j], lo = acc[j], junk16 = acc[j], junk32 = acc[j];
        permlane16_swap(junk16, mid);
        permlane32_swap(junk32, lo);
        acc[j] = (acc[j] + mid) + lo;
    }
    if (g == 0) {
#pragma unroll
        for (int j = 0; j < NT; ++j) part[(((size_t)pt * nsl + s) * 16 + n) * TP + j] = acc[j];
    }
}

// A fragments of a slice's 16 blocks: lane l holds row m = l % 16 (piece m / 4 of
// token m % 4; rows 12..15 and tokens >= NT are zero) at k = 8 (l / 16) .. + 7 of
// each block.  x is small and shared: its loads hit in L2.
template <int NT>
__device__ __forceinline__ void mfma_afrag(const float* __restrict__ x, const int64_t (&xoff)[NT], int k0, int cols,
                                           int lane, int g, V4 (&afrag)[16]) {
    const int am = lane & 15, ap = am >> 2, at = am & 3;
    const bool arow = ap < 3 && at < NT;
    int64_t xo = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) xo = at == t ? xoff[t] : xo;
    const float m1 = ap >= 1 ? 1.0f : 0.0f, m2 = ap >= 2 ? 1.0f : 0.0f;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
        const int kb = k0 + 32 * b + 8 * g;
        const bool ok = arow && kb < cols;
        const float4* px = reinterpret_cast<const float4*>(x + (ok ? xo + kb : 0));
        const float4 u = px[0], v = px[1];
        const float xs[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo16 = x_piece(xs[2 * i], m1, m2), hi16 = x_piece(xs[2 * i + 1], m1, m2);
            afrag[b][i] = ok ? lo16 | (hi16 << 16) : 0u;
        }
        if (b == 7) __builtin_amdgcn_sched_barrier(0);  // two rounds of x loads: bounds live registers
    }
}

template <int NT, class Out>
__device__ __forceinline__ void mfma_rows_q8(const uint8_t* __restrict__ W, int64_t row_bytes, int cols, int nsl,
                                             const float* __restrict__ x, const int64_t (&xoff)[NT], int64_t row_begin,
                                             int64_t row_end, Out out) {
    constexpr int FMT = QG_FMT_Q8_0;
    constexpr int ST = 16;
    using S = StreamShape<FMT, ST>;
    constexpr int L = S::kLoads;
    constexpr int TP = pad_pow2(NT);
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps buffer descriptors scalar
    const int nw = blockDim.x >> 6;
    const int n = lane & 15;   // B / D column: weight row in the tile
    const int g = lane >> 4;   // k group of A / B; D row group
    const int s = wave % nsl;
    const int rg = wave / nsl;
    const int RG = nw / nsl;
    const int k0 = s * kSlice;
    const int ntiles = (int)((row_end - row_begin + ST - 1) / ST);
    uint8_t* buf = smem + wave * S::kBufBytes;
    float* part = reinterpret_cast<float*>(smem + nw * S::kBufBytes);  // [tiles][nsl][16][TP]

    const int64_t rest = row_bytes - (int64_t)s * S::kChunks * 16;
    const int cs = rest / 16 < S::kChunks ? (int)(rest / 16) : S::kChunks;
    const int nblk = (int)(rest / 34) < 16 ? (int)(rest / 34) : 16;  // blocks of this slice
    const int sbase = s * S::kChunks * 16;
    const int rbytes = (int)row_bytes;  // 16 rows of a tile fit in int32 (checked on the host)

    V4 afrag[16];
    mfma_afrag<NT>(x, xoff, k0, cols, lane, g, afrag);

    // one tile in flight per wave in registers (the A fragments and the four
    // accumulators leave no room for a second); a CU's waves together keep
    // enough bytes in flight
    V4 ra[L];
    mfma_issue(W, rbytes, row_begin, row_end, ntiles, rg, lane, cs, sbase, ra);
    for (int t = rg; t < ntiles; t += RG)
        mfma_tile_q8<NT>(W, rbytes, row_begin, row_end, ntiles, t, RG, cs, sbase, ra, buf, part, afrag, lane, n, g, s,
                         nsl, nblk, t);
    __syncthreads();
    const int nrows = (int)(row_end - row_begin);
    for (int o = tid; o < nrows * NT; o += blockDim.x) {
        const int rr = o / NT, t = o % NT;
        const int tl = rr / ST, nn = rr % ST;
        const float* base = part + (((size_t)tl * nsl) * 16 + nn) * TP + t;
        float sum = base[0];
        for (int w = 1; w < nsl; ++w) sum = sum + base[(size_t)w * 16 * TP];
        out(t, row_begin + rr, sum);
    }
}

// Persistent form of the matrix-core kernel: one workgroup per CU takes a
// balanced contiguous range of 16-row tiles, computes its A fragments once, and
// streams the whole range.  Partial sums go to one of two chunk buffers of C
// tiles; the last wave to finish a chunk (an LDS arrival counter) sums the
// slices and writes y while the others go on, so no wave waits at a barrier.
// A wave may start filling a chunk buffer only after the chunk that last used
// it has been summed (a generation count per buffer; the wave that sums it is
// never waiting on anything, so every wait ends).
template <int NT, class Out>
__device__ __forceinline__ void mfma_persist_q8(const uint8_t* __restrict__ W, int64_t rows, int64_t row_bytes, int cols,
                                                int nsl, int C, const float* __restrict__ x, const int64_t (&xoff)[NT],
                                                Out&& out) {
    constexpr int FMT = QG_FMT_Q8_0;
    constexpr int ST = 16;
    using S = StreamShape<FMT, ST>;
    constexpr int L = S::kLoads;
    constexpr int TP = pad_pow2(NT);
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = blockDim.x >> 6;  // == nsl: one wave per k slice
    const int n = lane & 15, g = lane >> 4;
    const int s = wave;
    const int64_t TT = (rows + ST - 1) / ST;
    const int64_t t0 = (int64_t)blockIdx.x * TT / gridDim.x, t1 = (int64_t)(blockIdx.x + 1) * TT / gridDim.x;
    const int64_t row_begin = t0 * ST;
    const int64_t row_end = t1 * ST < rows ? t1 * ST : rows;
    const int ntiles = (int)(t1 - t0);
    uint8_t* buf = smem + wave * S::kBufBytes;
    float* part = reinterpret_cast<float*>(smem + nw * S::kBufBytes);            // [2][C][nsl][16][TP]
    int* ctl = reinterpret_cast<int*>(part + (size_t)2 * C * nsl * 16 * TP);     // arrivals[2], generation[2]
    if (tid < 4) ctl[tid] = 0;
    __syncthreads();

    const int64_t rest = row_bytes - (int64_t)s * S::kChunks * 16;
    const int cs = rest / 16 < S::kChunks ? (int)(rest / 16) : S::kChunks;
    const int nblk = (int)(rest / 34) < 16 ? (int)(rest / 34) : 16;
    const int sbase = s * S::kChunks * 16;
    const int rbytes = (int)row_bytes;

    V4 afrag[16];
    mfma_afrag<NT>(x, xoff, s * kSlice, cols, lane, g, afrag);
    V4 ra[L];
    mfma_issue(W, rbytes, row_begin, row_end, ntiles, 0, lane, cs, sbase, ra);
    for (int c = 0; c * C < ntiles; ++c) {
        const int pb = c & 1;
        if (c >= 2) {  // chunk c - 2 (same buffer) must have been summed
            while (__atomic_load_n(&ctl[2 + pb], __ATOMIC_RELAXED) < (c >> 1)) __builtin_amdgcn_s_sleep(1);
            lds_acquire();
        }
        const int tend = (c + 1) * C < ntiles ? (c + 1) * C : ntiles;
        for (int t = c * C; t < tend; ++t)
            mfma_tile_q8<NT>(W, rbytes, row_begin, row_end, ntiles, t, 1, cs, sbase, ra, buf, part, afrag, lane, n, g,
                             s, nsl, nblk, pb * C + (t - c * C));
        lds_release();  // the partials, then the arrival
        int last = 0;
        if (lane == 0) last = __atomic_fetch_add(&ctl[pb], 1, __ATOMIC_RELAXED) == nw - 1;
        last = __shfl(last, 0, 64);
        if (last) {  // every wave's partials of chunk c are in: sum the slices in order
            lds_acquire();
            const int64_t r0 = row_begin + (int64_t)c * C * ST;
            const int nr = (int)((row_end - r0) < (int64_t)C * ST ? (row_end - r0) : (int64_t)C * ST);
            for (int o = lane; o < nr * NT; o += 64) {
                const int rr = o / NT, t = o % NT;
                const float* base = part + (((size_t)(pb * C + rr / ST) * nsl) * 16 + rr % ST) * TP + t;
                float sum = base[0];
                for (int w = 1; w < nsl; ++w) sum = sum + base[(size_t)w * 16 * TP];
                out(t, r0 + rr, sum);
            }
            lds_release();  // the partials are read
            if (lane == 0) {
                __atomic_store_n(&ctl[pb], 0, __ATOMIC_RELAXED);
                __atomic_fetch_add(&ctl[2 + pb], 1, __ATOMIC_RELAXED);
            }
        }
    }
    wait_vmcnt<0>();  // the last (empty) prefetch returns before the wave ends
}

// ------------------------- matrix cores on the LDS-DMA ring, 256-wide slices (kind 8)
// The half-slice kernel's work split (one wave per 256-wide k slice, every
// wave walks the workgroup's rows) with 16-row tiles contracted on the matrix
// cores: per 32-weight block of a tile, one v_mfma_f32_16x16x32_bf16 with
//   A = the slice's x split exactly into three bf16 pieces (row m = 4p + t holds
//       piece p of token t; rows with t >= T and rows 12..15 are zero), and
//   B = the block's codes of the 16 rows as bf16 (exact; Q4_0 as 16 (c - 8)),
// so every product is exact; lane l gets the block's sums for row l % 16, which
// it scales by that row's d and accumulates in fp32 (BF16: the matrix core
// accumulates straight into the running sum).  At the end of a tile the three
// pieces of each token are added in a fixed order.  A token's rows of A never
// touch another token's, so its bits do not depend on T; the work per tile does
// not depend on T either.
// The split is done once per wave and cooperatively: each lane splits four x
// values of every token and the pieces reach the fragment layout through LDS
// (each lane loading the 64 values its fragments hold straight from memory
// instead multiplies x's cache traffic by 16 and measured 20-50 % slower).
// Each wave keeps one tile in flight, refilled as soon as the tile's bytes are
// in registers; measured on 10240 x 2560, a second tile in flight or a refill
// after the math is slower (the vector-ALU kernels behave alike).
// A tile is R groups of 16 rows (R = 2: twice the bytes in flight per wave, for
// the formats with short rows) of a slice of H 256-wide halves (H = 2: 512-wide
// slices, 16 blocks a wave, for rows of more than twelve 256-wide slices).
template <int FMT, int R = 1, int H = 1>
struct MxShape {
    static constexpr int kChunks = StreamFmt<FMT>::kChunks / 2 * H;      // 16-byte chunks of a row slice
    static constexpr int kRows = 16 * R;                                  // rows of a tile
    static constexpr int kSlot = kRows * kChunks * 16;                    // 16 rows: 4352, 2304, 8192 B
    static constexpr int kLoads = (kRows * kChunks + 63) / 64;            // 16 rows: 5, 3, 8
    static constexpr int kLastLanes = kRows * kChunks - 64 * (kLoads - 1);  // lanes of the last load (16 rows: 16, 16, 64)
    static constexpr int kBlockBytes = FMT == QG_FMT_Q8_0 ? 34 : FMT == QG_FMT_Q4_0 ? 18 : 64;
};

// Cache policy of the dense matrix-core kinds' weight loads, by format (measured:
// streaming takes 0.1-0.5 µs off the Q4_0 and BF16 8192 x 2560 calls and adds
// 0.1-0.4 µs to the Q8_0 ones; the split the persistent kind uses adds 0.5-1.2 µs
// to every one of them, whose few tiles per wave leave no room for twice the load
// instructions).
template <int FMT>
constexpr int kDensePolicy = FMT == QG_FMT_Q8_0 ? kDefaultPolicy : kStreamPolicy;

// One tile of the wave's slice into its slot: lane l of load k fetches chunk
// 64 k + l (row / chunk of the slice); lanes past the tile's last chunk do not
// load, so the slot is exactly the tile's bytes; rows past the range are
// outside the descriptor and read as zeros.
template <int FMT, int R = 1, int H = 1, int POLICY = kDefaultPolicy>
__device__ __forceinline__ void mx_issue(const uint8_t* __restrict__ W, int64_t row_bytes, int64_t row_begin,
                                         int64_t row_end, int ntiles, int t, const int (&off)[MxShape<FMT, R, H>::kLoads],
                                         uint8_t* slot, int lane) {
    static_assert(POLICY != kSplitPolicy, "the dense kinds keep one policy per load");
    using M = MxShape<FMT, R, H>;
    const bool live = t < ntiles;
    const int64_t r0 = row_begin + (int64_t)(live ? t : 0) * M::kRows;
    const int64_t rows_here = row_end - r0 < M::kRows ? row_end - r0 : M::kRows;
    const int num = live ? (int)(rows_here * row_bytes) : 0;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(W + r0 * row_bytes), (short)0, num, kBufferRsrcWord3);
#pragma unroll
    for (int k = 0; k < M::kLoads - 1; ++k) load_lds16<POLICY>(rsrc, slot + 1024 * k, off[k]);
    if (M::kLastLanes == 64 || lane < M::kLastLanes)
        load_lds16<POLICY>(rsrc, slot + 1024 * (M::kLoads - 1), off[M::kLoads - 1]);
}

// Byte q of the 12-byte window w[3] as an fp32 (signed).
__device__ __forceinline__ uint32_t mx_byte_f32(const uint32_t (&w)[3], int q) {
    return __builtin_bit_cast(uint32_t, (float)(int32_t)(int8_t)(w[q >> 2] >> (8 * (q & 3))));
}

// The bytes of block b that lane (row n, k group g) needs, as read from the
// LDS: Q8_0 / Q4_0 blocks of an even index start 2 bytes past a dword, so their
// codes are read as an aligned 12-byte window whose bytes 2..9 are taken (odd
// blocks: an 8-byte window); BF16: the 16 bytes of the lane's 8 codes.  `d`
// holds the block's fp16 scale bits.
struct MxRaw {
    uint32_t w[4];
    uint32_t d;
};

template <int FMT>
__device__ __forceinline__ MxRaw mx_braw(const uint8_t* rowp, int b, int g) {
    using M = MxShape<FMT>;
    MxRaw r;
    if constexpr (FMT == QG_FMT_BF16) {
        const U4a q = *reinterpret_cast<const U4a*>(rowp + M::kBlockBytes * b + 16 * g);
        r.w[0] = q.v[0]; r.w[1] = q.v[1]; r.w[2] = q.v[2]; r.w[3] = q.v[3];
        r.d = 0;
    } else {
        const uint8_t* blk = rowp + M::kBlockBytes * b;
        // Q8_0: the lane's codes are bytes 8g..8g+7 of the block's 32; Q4_0: the low
        // (g < 2) or high (g >= 2) nibbles of code bytes 8(g & 1)..+7, i.e. codes 8g..8g+7
        const int cb = FMT == QG_FMT_Q8_0 ? 8 * g : 8 * (g & 1);
        const int sh = (b & 1) ? 0 : 2;  // where the codes start in the window
        const uint32_t* p = reinterpret_cast<const uint32_t*>(blk + 2 + cb - sh);
        r.w[0] = p[0]; r.w[1] = p[1]; r.w[2] = sh ? p[2] : 0u; r.w[3] = 0u;
        r.d = *reinterpret_cast<const uint16_t*>(blk);
    }
    return r;
}

// The B fragment of block b from its bytes: 8 codes as bf16 pairs, and the
// block's scale (Q4_0: d / 16; BF16: 1).
template <int FMT>
__device__ __forceinline__ V4 mx_bconv(const MxRaw& raw, int b, int g, float& d) {
    V4 r;
    if constexpr (FMT == QG_FMT_BF16) {
        r[0] = raw.w[0]; r[1] = raw.w[1]; r[2] = raw.w[2]; r[3] = raw.w[3];
        d = 1.0f;
    } else {
        const int sh = (b & 1) ? 0 : 2;
        uint32_t w[3] = {raw.w[0], raw.w[1], raw.w[2]};
        if constexpr (FMT == QG_FMT_Q4_0) {
            // nibble c -> the signed byte 16 (c - 8): flip bit 3, move the nibble to the top
            const int ns = g >= 2 ? 0 : 4;
#pragma unroll
            for (int i = 0; i < 3; ++i) w[i] = ((w[i] << ns) & 0xF0F0F0F0u) ^ 0x80808080u;
        }
        uint32_t f[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) f[q] = mx_byte_f32(w, q + sh);
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q] = __builtin_amdgcn_perm(f[2 * q + 1], f[2 * q], 0x07060302u);
        const float dv = half_bits_to_float((uint16_t)raw.d);
        d = FMT == QG_FMT_Q4_0 ? dv * 0.0625f : dv;
    }
    return r;
}

// The B fragment of block b for lane (row n, k group g) and the block's scale.
template <int FMT>
__device__ __forceinline__ V4 mx_bfrag(const uint8_t* rowp, int b, int g, float& d) {
    return mx_bconv<FMT>(mx_braw<FMT>(rowp, b, g), b, g, d);
}

// The wave's first tile of a row range, issued ahead of the rest of the
// prologue (the grouped kernel's scan of the ids); mx_rows<..., PRE = true> then
// does not issue it again.
template <int FMT, int R>
__device__ __forceinline__ void mx_prefetch(const uint8_t* __restrict__ W, int64_t row_bytes, int nsl, int64_t row_begin,
                                            int64_t row_end) {
    using M = MxShape<FMT, R>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int s = wave % nsl, rg = wave / nsl;
    const int ntiles = (int)((row_end - row_begin + M::kRows - 1) / M::kRows);
    int off[M::kLoads];
#pragma unroll
    for (int k = 0; k < M::kLoads; ++k) {
        const int j = 64 * k + lane;
        const int r = j / M::kChunks, c = j % M::kChunks;
        off[k] = r < M::kRows ? (int)(r * row_bytes) + s * M::kChunks * 16 + 16 * c : kNoLoad;
    }
    mx_issue<FMT, R>(W, row_bytes, row_begin, row_end, ntiles, rg, off, smem + wave * M::kSlot, lane);
}

// x of token t of the wave's slice: lane l holds k = 4 l .. 4 l + 3 of the
// slice's 256-wide half h in xv[t][h] (one coalesced 1 KB row per token and
// half, loaded by the caller).
template <int FMT, int NT, int H = 1>
__device__ __forceinline__ void mx_load_x(const float* __restrict__ x, const int64_t (&xoff)[NT], int nsl,
                                          float4 (&xv)[NT][H]) {
    int rg, s;
    small_divmod((int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nsl, rg, s);
    const int k0 = s * (kHalfSlice * H);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int h = 0; h < H; ++h)
            xv[t][h] = *reinterpret_cast<const float4*>(x + xoff[t] + k0 + kHalfSlice * h + 4 * (threadIdx.x & 63));
}

// GATHER: the rows are ids[row_begin .. row_end) of W's `wrows` rows (at most 128 a
// workgroup, W under 2 GB): every wave holds the workgroup's ids in registers (id j
// in lane j % 64 of register j / 64) and each load lane takes its row's id from the
// lane that holds it; an id outside [0, wrows) loads nothing (the caller writes NaN).
template <int FMT, int NT, int R, bool PRE = false, int H = 1, bool GATHER = false, int POLICY = kDefaultPolicy,
          class Out>
__device__ __forceinline__ void mx_rows(const uint8_t* __restrict__ W, int64_t row_bytes, int nsl,
                                        const float4 (&xv)[NT][H], int64_t row_begin, int64_t row_end, int nw,
                                        Out&& out, const int32_t* __restrict__ ids = nullptr, int64_t wrows = 0) {
    using M = MxShape<FMT, R, H>;
    constexpr int NB = 8 * H;  // blocks of a wave's slice
    static_assert(!GATHER || (R == 1 && !PRE), "a gathered tile is 16 rows, issued here");
    constexpr int RT = M::kRows;
    constexpr int TP = pad_pow2(NT);
    constexpr int L = M::kLoads;
    constexpr int REG = 1536;  // per wave: one token's bf16 pieces [8 blocks][4 groups][3 pieces] x 16 B
    // a lane's rows of D past the first NJ belong to no token (A's rows of tokens >=
    // NT are zero): their scalings and piece sums are skipped and they stay 0
    constexpr int NJ = NT < 4 ? NT : 4;
    // three or four tokens: A's row 4t + p holds piece p of token t (token-major), so a
    // lane holds the three pieces of one token, scales three rows of D per block and
    // adds its pieces in place; one or two: row 4p + t (piece-major), so a lane scales
    // only NJ rows and the pieces meet across lanes.  Either way a token's arithmetic
    // is the same, and so are its bits.  The gathered rows stay piece-major: their
    // id exchange leaves no registers for the token-major form at three tokens (it
    // spilled and ran 47 µs against 38 on a 32,768-row subset).
    constexpr bool TM = NT >= 3 && !GATHER;
    constexpr int NS = TM ? 3 : NJ;  // rows of D a lane scales
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps descriptors and M0 scalar
    const int n = lane & 15, g = lane >> 4;
    int s, rg, RG, rest;
    small_divmod(wave, nsl, rg, s);
    small_divmod(nw, nsl, RG, rest);
    const int ntiles = (int)((row_end - row_begin + RT - 1) / RT);
    uint8_t* slot = smem + wave * M::kSlot;
    uint8_t* reg = smem + nw * M::kSlot + wave * REG;
    float* part = reinterpret_cast<float*>(smem + nw * (M::kSlot + REG));  // [tiles][nsl][RT rows][TP]

    int off[L];
#pragma unroll
    for (int k = 0; k < L; ++k) {
        const int j = 64 * k + lane;
        const int r = j / M::kChunks, c = j % M::kChunks;
        off[k] = r < RT ? (GATHER ? 0 : (int)(r * row_bytes)) + s * M::kChunks * 16 + 16 * c : kNoLoad;
    }
    int my_id0 = -1, my_id1 = -1;
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void*)W, (short)0, GATHER ? (int)(wrows * row_bytes) : 0, kBufferRsrcWord3);
    if constexpr (GATHER) {
        const int nsel = (int)(row_end - row_begin);
        my_id0 = lane < nsel ? ids[row_begin + lane] : -1;
        my_id1 = 64 + lane < nsel ? ids[row_begin + 64 + lane] : -1;
    }
    auto issue = [&](int t) __attribute__((always_inline)) {
        if constexpr (GATHER) {
            // every lane takes part in the exchanges (a lane outside a load's exec
            // would hand its neighbours nothing), then the loads
            int idk[L];
#pragma unroll
            for (int k = 0; k < L; ++k) {
                const int src = t * 16 + (64 * k + lane) / M::kChunks;  // tiles 0..3 read ids 0..63
                idk[k] = __shfl(t < 4 ? my_id0 : my_id1, src & 63, 64);
            }
#pragma unroll
            for (int k = 0; k < L; ++k) {
                if (k == L - 1 && M::kLastLanes < 64 && lane >= M::kLastLanes) break;
                const int r = (64 * k + lane) / M::kChunks;
                const int src = t * 16 + r;
                const int id = idk[k];
                const bool live = t < ntiles && r < 16 && src < (int)(row_end - row_begin) && id >= 0 && id < wrows;
                load_lds16(wr, slot + 1024 * k, live ? (int)(id * row_bytes) + off[k] : kNoLoad);
            }
        } else {
            mx_issue<FMT, R, H, POLICY>(W, row_bytes, row_begin, row_end, ntiles, t, off, slot, lane);
        }
    };
    // the wave's first tile, unless PRE has it on its way already (x is older)
    if constexpr (!PRE) issue(rg);

    // split, one token and 256-wide half at a time through the wave's region: piece
    // p of x[t][k] goes to the 16-byte fragment (block k / 32, group (k % 32) / 8,
    // piece p), which the lane of A's row (4p + t, or 4t + p) and group (k % 32) / 8
    // then reads.
    // A wave's LDS operations take effect in program order, so the next round's
    // writes land after this round's reads.
    V4 afrag[NB];
    {
        const int b = lane >> 3, gg = (lane & 7) >> 1, half = (lane & 1) * 8;
        const int am = lane & 15, ap = TM ? (am & 3) : (am >> 2), at = TM ? (am >> 2) : (am & 3);
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) afrag[bb] = V4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int hx = 0; hx < H; ++hx)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float vv[4] = {xv[t][hx].x, xv[t][hx].y, xv[t][hx].z, xv[t][hx].w};
            uint32_t pc[3][4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // hi = x with its low 16 bits cleared, mid = the same of x - hi, lo = x - hi - mid:
                // exact (x has 24 significant bits), and each piece is exactly a bf16
                const uint32_t v = __builtin_bit_cast(uint32_t, vv[q]);
                const float r1 = vv[q] - __builtin_bit_cast(float, v & 0xFFFF0000u);
                const uint32_t u1 = __builtin_bit_cast(uint32_t, r1);
                const float r2 = r1 - __builtin_bit_cast(float, u1 & 0xFFFF0000u);
                pc[0][q] = v;
                pc[1][q] = u1;
                pc[2][q] = __builtin_bit_cast(uint32_t, r2);
            }
#pragma unroll
            for (int p = 0; p < 3; ++p) {
                uint2 w2;
                w2.x = __builtin_amdgcn_perm(pc[p][1], pc[p][0], 0x07060302u);
                w2.y = __builtin_amdgcn_perm(pc[p][3], pc[p][2], 0x07060302u);
                *reinterpret_cast<uint2*>(reg + b * 192 + (gg * 3 + p) * 16 + half) = w2;
            }
            if (ap < 3 && at == t) {
#pragma unroll
                for (int bb = 0; bb < 8; ++bb)
                    afrag[8 * hx + bb] = *reinterpret_cast<const V4*>(reg + bb * 192 + (g * 3 + ap) * 16);
            }
        }
    }

    const int mine = ntiles > rg ? (RG == 1 ? ntiles - rg : (ntiles - rg + RG - 1) / RG) : 0;
    const uint8_t* rowp = slot + n * (M::kChunks * 16);
    for (int i = 0; i < mine; ++i) {
        const int t = rg + i * RG;
        wait_vmcnt<0>();  // the slot holds tile t
        MxRaw raw[R][NB];
#pragma unroll
        for (int h = 0; h < R; ++h)
#pragma unroll
            for (int b = 0; b < NB; ++b) raw[h][b] = mx_braw<FMT>(rowp + 16 * h * (M::kChunks * 16), b, g);
        wait_lgkmcnt0();  // the tile is in registers: the slot takes the next one
        if (i + 1 < mine) issue(t + RG);
#pragma unroll
        for (int h = 0; h < R; ++h) {
            F4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float dq;
                const V4 bq = mx_bconv<FMT>(raw[h][b], b, g, dq);
                if constexpr (FMT == QG_FMT_BF16) {
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(BF8, afrag[b]),
                                                                  __builtin_bit_cast(BF8, bq), acc, 0, 0, 0);
                } else {
                    const F4 z = {0.0f, 0.0f, 0.0f, 0.0f};
                    const F4 dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(BF8, afrag[b]),
                                                                          __builtin_bit_cast(BF8, bq), z, 0, 0, 0);
#pragma unroll
                    for (int j = 0; j < NS; ++j) acc[j] = __builtin_fmaf(dq, dd[j], acc[j]);
                }
            }
            if constexpr (TM) {  // the lane's token g: (hi + mid) + lo
                const float tok = (acc[0] + acc[1]) + acc[2];
                if (g < NT) part[(((size_t)t * nsl + s) * RT + 16 * h + n) * TP + g] = tok;
            } else {
                // token j's pieces sit in lanes n (hi), n + 16 (mid), n + 32 (lo): (hi + mid) + lo
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    float mid = acc[j], lo = acc[j], junk16 = acc[j], junk32 = acc[j];
                    permlane16_swap(junk16, mid);
                    permlane32_swap(junk32, lo);
                    acc[j] = (acc[j] + mid) + lo;
                }
                if (lane < 16) {
                    float* pp = part + (((size_t)t * nsl + s) * RT + 16 * h + n) * TP;
#pragma unroll
                    for (int j = 0; j < TP; ++j) pp[j] = acc[j];
                }
            }
        }
    }
    wait_vmcnt<0>();  // a wave with no tile still drains its empty load
    __syncthreads();
    // every output of the workgroup: sum the slices' partials in slice order
    const int nrows = (int)(row_end - row_begin);
    for (int o = tid; o < nrows * NT; o += blockDim.x) {
        const int rr = o / NT, tk = o % NT;
        const float* base = part + ((size_t)(rr / RT) * nsl * RT + rr % RT) * TP + tk;
        float sum = base[0];
        for (int w = 1; w < nsl; ++w) sum = sum + base[(size_t)w * RT * TP];
        out(tk, row_begin + rr, sum);
    }
}

// ----------------- persistent matrix cores on the LDS-DMA ring, 512-wide slices (kind 9)
// For long matrices (the LM head): one workgroup per CU walks a contiguous range
// of 16-row tiles, one wave per 512-wide k slice (16 blocks), with the
// arithmetic of kind 8 per block.  A wave's slot holds one 16-row tile of its
// slice; its bytes are read raw into registers (the conversion to bf16 waits
// for the MFMAs, which keeps the registers within three waves per SIMD) and the
// slot is refilled at once.  Before the first tile the slot stages x and its
// bf16 pieces (two rounds of eight blocks), so the A fragments cost one pass
// per wave and no LDS of their own.  Partial sums go to two chunk buffers of C
// tiles; one more wave, which streams nothing, waits for each chunk's arrivals
// (an LDS counter), adds the slices in slice order and stores the outputs, so no
// streaming wave ever stops its stream to sum (a summing wave that also streams
// cannot overlap the sums with its tile in flight: the compiler waits for the
// load into LDS before the protocol's LDS reads).  A wave reuses a chunk buffer
// only once its previous chunk has been summed (a generation count); the summing
// wave waits only for arrivals that every streaming wave makes, so every wait ends.
template <int FMT>
struct MxpShape {
    static constexpr int kChunks = StreamFmt<FMT>::kChunks;              // 16-byte chunks of a row slice: 34, 18, 64
    static constexpr int kRow = 16 * kChunks;                             // 544, 288, 1024 B
    static constexpr int kTile = 16 * kRow;                               // 8704, 4608, 16384 B
    static constexpr int kSlot = kTile > 8192 ? kTile : 8192;             // x of four tokens fits too
    static constexpr int kLoads = (16 * kChunks + 63) / 64;               // 9, 5, 16
    static constexpr int kLastLanes = 16 * kChunks - 64 * (kLoads - 1);   // 32, 32, 64
};

// Cache policy of the persistent kind's weight loads, by format (measured): Q8_0
// splits (its 544-byte row pieces share only their two end lines); Q4_0's
// 288-byte pieces share most of their lines, and there streaming every load ran
// 0.3-4 µs faster than the split on 151,936 x 3,584 and 248,320 x 5,120; BF16's
// 1 KB pieces share none.
template <int FMT>
constexpr int kPersistPolicy = FMT == QG_FMT_Q8_0 ? kSplitPolicy : kStreamPolicy;

// 16-row tile t of the wave's slice into its slot: lane l of load k fetches
// chunk 64 k + l (row / chunk of the row slice); rows past the range are
// outside the descriptor and read as zeros.  The matrices this kind serves are
// beyond the last-level cache: the loads stream (Q8_0: but for the chunks in
// lines shared with a neighbouring piece, `shm`).
template <int FMT>
__device__ __forceinline__ void mxp_issue(const uint8_t* __restrict__ W, int64_t row_bytes, int64_t row_begin,
                                          int64_t row_end, int t, const int (&off)[MxpShape<FMT>::kLoads],
                                          uint8_t* slot, int lane, uint32_t shm) {
    using M = MxpShape<FMT>;
    const int64_t r0 = row_begin + (int64_t)t * 16;
    const int64_t rows_here = row_end - r0 < 16 ? row_end - r0 : 16;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(W + r0 * row_bytes), (short)0, (int)(rows_here * row_bytes), kBufferRsrcWord3);
#pragma unroll
    for (int k = 0; k < M::kLoads - 1; ++k) load_w16<kPersistPolicy<FMT>>(rsrc, slot + 1024 * k, off[k], (shm >> k) & 1u);
    if (M::kLastLanes == 64 || lane < M::kLastLanes)
        load_w16<kPersistPolicy<FMT>>(rsrc, slot + 1024 * (M::kLoads - 1), off[M::kLoads - 1],
                                      (shm >> (M::kLoads - 1)) & 1u);
}

// The MFMAs of the 16 blocks of one tile, from their bytes: acc += scale *
// (pieces x codes) per block, in block order.
template <int FMT, int NT>
__device__ __forceinline__ void mxp_math(const V4 (&afrag)[16], const MxRaw (&raw)[16], int g, F4& acc) {
    // rows of D that carry a token (the rest stay 0); with three or four tokens A is
    // token-major (row 4t + p) and a lane scales its token's three pieces
    constexpr int NJ = NT >= 3 ? 3 : NT;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
        float dq;
        const V4 bq = mx_bconv<FMT>(raw[b], b, g, dq);
        if constexpr (FMT == QG_FMT_BF16) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(BF8, afrag[b]),
                                                          __builtin_bit_cast(BF8, bq), acc, 0, 0, 0);
        } else {
            const F4 z = {0.0f, 0.0f, 0.0f, 0.0f};
            const F4 dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(BF8, afrag[b]),
                                                                  __builtin_bit_cast(BF8, bq), z, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[j] = __builtin_fmaf(dq, dd[j], acc[j]);
        }
    }
}

// The partial sums of one row for every token, read or written at once.
template <int N>
struct alignas(4 * N) Vec {
    float v[N];
};

template <int FMT, int NT, class Out>
__device__ __forceinline__ void mxp_rows(const uint8_t* __restrict__ W, int64_t rows, int64_t row_bytes, int cols,
                                         int nsl, int C, const float* __restrict__ x, Out&& out) {
    using M = MxpShape<FMT>;
    constexpr int TP = pad_pow2(NT);
    constexpr int L = M::kLoads;
    static_assert(NT * 2048 <= M::kSlot && 1536 * NT <= M::kSlot, "x and its pieces are staged in the slot");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = nsl;                // streaming waves: one per k slice
    const bool summer = wave == nsl;   // the workgroup's last wave sums the chunks
    const int n = lane & 15, g = lane >> 4;
    const int s = wave;
    const int k0 = s * kSlice;
    const int64_t TT = (rows + 15) / 16;
    const int64_t t0 = (int64_t)blockIdx.x * TT / gridDim.x, t1 = (int64_t)(blockIdx.x + 1) * TT / gridDim.x;
    const int64_t row_begin = t0 * 16;
    const int64_t row_end = t1 * 16 < rows ? t1 * 16 : rows;
    const int ntiles = (int)(t1 - t0);
    uint8_t* slot = smem + (summer ? 0 : wave) * M::kSlot;
    float* part = reinterpret_cast<float*>(smem + nw * M::kSlot);              // [2][C][nsl][16][TP]
    // arrivals[2], generation[2]: an LDS object of their own, so the compiler can see that
    // reading them never depends on the tile loads into the dynamic LDS in flight
    __shared__ int ctl[4];
    if (tid < 4) ctl[tid] = 0;

    int off[L];
#pragma unroll
    for (int k = 0; k < L; ++k) {
        const int j = 64 * k + lane;
        const int r = j / M::kChunks, c = j % M::kChunks;
        off[k] = r < 16 ? (int)(r * row_bytes) + s * M::kRow + 16 * c : kNoLoad;
    }
    // tiles lie 16 rows apart: a multiple of 128 bytes for every Q8_0 / Q4_0 / BF16
    // row of whole 512-wide slices, so one mask serves them all
    const uint32_t shm = shared_line_mask<L>((uint64_t)(uintptr_t)W + (uint64_t)row_begin * (uint64_t)row_bytes +
                                                 (uint64_t)s * M::kRow,
                                             row_bytes, M::kChunks, 16, lane);
    // x of the slice into the slot (token t at 2048 t), then into registers: lane
    // l takes k = 4 l .. 4 l + 3 of each 256-wide half (the summing wave has no
    // slice: it skips the staging and keeps zero fragments)
    V4 afrag[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) afrag[b] = V4{0u, 0u, 0u, 0u};
    if (!summer) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const __amdgpu_buffer_rsrc_t xr =
                __builtin_amdgcn_make_buffer_rsrc((void*)(x + (int64_t)t * cols + k0), (short)0, 2048, kBufferRsrcWord3);
            load_lds16(xr, slot + 2048 * t, 16 * lane);
            load_lds16(xr, slot + 2048 * t + 1024, 16 * lane + 1024);
        }
        wait_vmcnt<0>();
        float4 xv[2][NT];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < NT; ++t) xv[h][t] = *reinterpret_cast<const float4*>(slot + 2048 * t + 1024 * h + 16 * lane);
        {
            const int b = lane >> 3, gg = (lane & 7) >> 1, half = (lane & 1) * 8;
            // A's row 4p + t (piece-major, one or two tokens) or 4t + p (token-major)
            const int am = lane & 15, ap = NT >= 3 ? (am & 3) : (am >> 2), at = NT >= 3 ? (am >> 2) : (am & 3);
            const bool arow = ap < 3 && at < NT;
            const int idx = arow ? (g * 3 * NT + ap * NT + at) * 16 : 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                wait_lgkmcnt0();  // the slot's previous contents are read by every lane
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const float vv[4] = {xv[h][t].x, xv[h][t].y, xv[h][t].z, xv[h][t].w};
                    uint32_t pc[3][4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t v = __builtin_bit_cast(uint32_t, vv[q]);
                        const float r1 = vv[q] - __builtin_bit_cast(float, v & 0xFFFF0000u);
                        const uint32_t u1 = __builtin_bit_cast(uint32_t, r1);
                        const float r2 = r1 - __builtin_bit_cast(float, u1 & 0xFFFF0000u);
                        pc[0][q] = v;
                        pc[1][q] = u1;
                        pc[2][q] = __builtin_bit_cast(uint32_t, r2);
                    }
#pragma unroll
                    for (int p = 0; p < 3; ++p) {
                        uint2 w2;
                        w2.x = __builtin_amdgcn_perm(pc[p][1], pc[p][0], 0x07060302u);
                        w2.y = __builtin_amdgcn_perm(pc[p][3], pc[p][2], 0x07060302u);
                        *reinterpret_cast<uint2*>(slot + b * (192 * NT) + (gg * 3 * NT + p * NT + t) * 16 + half) = w2;
                    }
                }
                wait_lgkmcnt0();
#pragma unroll
                for (int bb = 0; bb < 8; ++bb) {
                    const V4 v = *reinterpret_cast<const V4*>(slot + bb * (192 * NT) + idx);
                    afrag[8 * h + bb] = arow ? v : V4{0u, 0u, 0u, 0u};
                }
            }
        }
    }
    wait_lgkmcnt0();  // the pieces are in registers: the slot takes the first tile
    __syncthreads();  // (also publishes the cleared control words)
    if (summer) {  // every chunk: wait for all slices' partials, sum them in slice order, store
        for (int c = 0; c * C < ntiles; ++c) {
            const int pb = c & 1;
            while (__atomic_load_n(&ctl[pb], __ATOMIC_RELAXED) < nw) __builtin_amdgcn_s_sleep(1);
            lds_acquire();
            const int64_t r0 = row_begin + (int64_t)c * C * 16;
            const int nr = (int)((row_end - r0) < (int64_t)C * 16 ? (row_end - r0) : (int64_t)C * 16);
            for (int rr = lane; rr < nr; rr += 64) {  // a lane per row, all tokens at once
                const float* base = part + (((size_t)(pb * C + rr / 16) * nsl) * 16 + rr % 16) * TP;
                Vec<TP> sum = *reinterpret_cast<const Vec<TP>*>(base);
                for (int w = 1; w < nsl; ++w) {
                    const Vec<TP> v = *reinterpret_cast<const Vec<TP>*>(base + (size_t)w * 16 * TP);
#pragma unroll
                    for (int tk = 0; tk < NT; ++tk) sum.v[tk] = sum.v[tk] + v.v[tk];
                }
#pragma unroll
                for (int tk = 0; tk < NT; ++tk) out(tk, r0 + rr, sum.v[tk]);
            }
            lds_release();  // the partials are read
            if (lane == 0) {
                __atomic_store_n(&ctl[pb], 0, __ATOMIC_RELAXED);
                __atomic_fetch_add(&ctl[2 + pb], 1, __ATOMIC_RELAXED);
            }
        }
        return;
    }
    if (ntiles > 0) mxp_issue<FMT>(W, row_bytes, row_begin, row_end, 0, off, slot, lane, shm);

    const uint8_t* rowp = slot + n * M::kRow;
    for (int c = 0; c * C < ntiles; ++c) {
        const int pb = c & 1;
        if (c >= 2) {  // chunk c - 2 (same buffer) must have been summed
            while (__atomic_load_n(&ctl[2 + pb], __ATOMIC_RELAXED) < (c >> 1)) __builtin_amdgcn_s_sleep(1);
            lds_acquire();
        }
        const int tend = (c + 1) * C < ntiles ? (c + 1) * C : ntiles;
        for (int t = c * C; t < tend; ++t) {
            wait_vmcnt<0>();  // the slot holds tile t
            MxRaw raw[16];
#pragma unroll
            for (int b = 0; b < 16; ++b) raw[b] = mx_braw<FMT>(rowp, b, g);
            wait_lgkmcnt0();  // the tile is in registers: the slot takes the next one
            if (t + 1 < ntiles) mxp_issue<FMT>(W, row_bytes, row_begin, row_end, t + 1, off, slot, lane, shm);
            F4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
            mxp_math<FMT, NT>(afrag, raw, g, acc);
            if constexpr (NT >= 3) {  // token-major: the lane's token g, (hi + mid) + lo in place
                const float tok = (acc[0] + acc[1]) + acc[2];
                if (g < NT) part[(((size_t)(pb * C + t - c * C) * nsl + s) * 16 + n) * TP + g] = tok;
            } else {
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    float mid = acc[j], lo = acc[j], junk16 = acc[j], junk32 = acc[j];
                    permlane16_swap(junk16, mid);
                    permlane32_swap(junk32, lo);
                    acc[j] = (acc[j] + mid) + lo;
                }
                if (lane < 16) {
                    float* pp = part + (((size_t)(pb * C + t - c * C) * nsl + s) * 16 + n) * TP;
#pragma unroll
                    for (int j = 0; j < TP; ++j) pp[j] = acc[j];
                }
            }
        }
        // publish this wave's partials of chunk c, then count the arrival
        lds_release();
        if (lane == 0) __atomic_fetch_add(&ctl[pb], 1, __ATOMIC_RELAXED);
    }
    wait_vmcnt<0>();
}

// ------------------------------------------------------ fused argmax over rows
// The LM-head step right after the mat-vec (the drafter's LM head in the mlxcel
// drafter-cost issue): per token, the row with the largest y and that y, with y
// never written.  A (value, row) pair is packed into one 64-bit key whose
// unsigned order is (value, then lower row first): the value's bits mapped to an
// order-preserving unsigned integer in the high half, 0xFFFFFFFF - row in the
// low half.  Each thread keeps its best key per token, each wave reduces its
// lanes' keys, and one 64-bit atomic max per wave and token merges workgroups;
// max is order-independent, so the result does not depend on scheduling.
__device__ __forceinline__ uint64_t argmax_key(float v, int64_t row) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)row);
}

template <int NT>
struct ArgmaxOut {
    uint64_t best[NT];
    __device__ ArgmaxOut() {
#pragma unroll
        for (int t = 0; t < NT; ++t) best[t] = 0;
    }
    __device__ void operator()(int t, int64_t row, float v) {
        const uint64_t k = argmax_key(v, row);
#pragma unroll
        for (int j = 0; j < NT; ++j)  // t varies across lanes: no dynamic indexing
            if (j == t && k > best[j]) best[j] = k;
    }
    // The workgroup's maximum of each token's key merged into work[t] by one
    // atomic per token: wave maxima by butterfly, then across waves through the
    // LDS.  Every thread of the workgroup calls it after its last use of the LDS
    // (which needs 8 * NT bytes per wave).  One atomic per workgroup instead of
    // one per wave: these 64-bit atomics are resolved past the XCDs' L2s, one
    // address at a time, and thousands of them per call cost tens of µs.
    __device__ void merge(unsigned long long* work) {
        extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
        unsigned long long* keys = reinterpret_cast<unsigned long long*>(smem);
        uint64_t k[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            k[t] = best[t];
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) {
                const uint32_t lo = __shfl_xor((uint32_t)k[t], m, 64), hi = __shfl_xor((uint32_t)(k[t] >> 32), m, 64);
                const uint64_t o = ((uint64_t)hi << 32) | lo;
                k[t] = o > k[t] ? o : k[t];
            }
        }
        const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
        __syncthreads();  // every wave is done with the LDS
        if ((threadIdx.x & 63) == 0) {
#pragma unroll
            for (int t = 0; t < NT; ++t) keys[wave * NT + t] = k[t];
        }
        __syncthreads();
        if ((int)threadIdx.x < NT) {
            unsigned long long m = 0;
            for (int w = 0; w < nw; ++w) {
                const unsigned long long o = keys[w * NT + threadIdx.x];
                m = o > m ? o : m;
            }
            if (m != 0) atomicMax(work + threadIdx.x, m);
        }
    }
};

__global__ void qgemv_argmax_init_kernel(unsigned long long* work, int T) {
    if ((int)threadIdx.x < T) work[threadIdx.x] = 0;
}

__global__ void qgemv_argmax_finish_kernel(const unsigned long long* work, int32_t* idx, float* val, int T) {
    const int t = threadIdx.x;
    if (t >= T) return;
    const uint64_t k = work[t];
    const uint32_t ord = (uint32_t)(k >> 32);
    const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
    idx[t] = (int32_t)(0xFFFFFFFFu - (uint32_t)k);
    val[t] = __builtin_bit_cast(float, u);
}

// ---------------------------------------------------------------- kernels
// The dense-path kernels take scalar arguments (not a struct): they can be
// preloaded into SGPRs at wave launch, so a wave issues its first loads without
// waiting on a kernel-argument load (nw: waves per workgroup, for the same reason).
template <int FMT, int T, int RB, bool ONE_SHOT>
__global__ void __launch_bounds__(64 * kMaxWaves)
qgemv_dense_kernel(const uint8_t* __restrict__ W, const float* __restrict__ x, float* __restrict__ y, int64_t rows,
                   int64_t row_bytes, int cols, int nslices, int rows_per_wg, int nw) {
    const int64_t row_begin = (int64_t)blockIdx.x * rows_per_wg;
    const int64_t row_end = row_begin + rows_per_wg < rows ? row_begin + rows_per_wg : rows;
    int64_t xoff[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xoff[t] = (int64_t)t * cols;
    gemv_rows<FMT, T, RB, ONE_SHOT>(W, row_bytes, cols, nslices, x, xoff, row_begin, row_end, nw,
                                    [=](int t, int64_t row, float v) { y[t * rows + row] = v; });
}

template <int FMT, int T, int ST>
__global__ void __launch_bounds__(64 * kMaxWaves)
qgemv_stream_kernel(const uint8_t* __restrict__ W, const float* __restrict__ x, float* __restrict__ y, int64_t rows,
                    int64_t row_bytes, int cols, int nslices, int rows_per_wg, int nw) {
    const int64_t row_begin = (int64_t)blockIdx.x * rows_per_wg;
    const int64_t row_end = row_begin + rows_per_wg < rows ? row_begin + rows_per_wg : rows;
    int64_t xoff[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xoff[t] = (int64_t)t * cols;
    stream_rows<FMT, T, ST>(W, row_bytes, cols, nslices, x, xoff, row_begin, row_end, nw,
                            [=](int t, int64_t row, float v) { y[t * rows + row] = v; });
}

template <int FMT, int T, int ST, int D, bool XSEP>
__global__ void __launch_bounds__(64 * kMaxWaves)
qgemv_dma_kernel(const uint8_t* __restrict__ W, const float* __restrict__ x, float* __restrict__ y, int64_t rows,
                 int64_t row_bytes, int cols, int nslices, int rows_per_wg, int nw) {
    const int64_t row_begin = (int64_t)blockIdx.x * rows_per_wg;
    const int64_t row_end = row_begin + rows_per_wg < rows ? row_begin + rows_per_wg : rows;
    int64_t xoff[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xoff[t] = (int64_t)t * cols;
    dma_rows<FMT, T, ST, D, XSEP>(W, row_bytes, cols, nslices, x, xoff, row_begin, row_end, nw,
                                  [=](int t, int64_t row, float v) { y[t * rows + row] = v; });
}

template <int FMT, int T, int D>
__global__ void __launch_bounds__(64 * kMaxWaves)
qgemv_half_kernel(const uint8_t* __restrict__ W, const float* __restrict__ x, float* __restrict__ y, int64_t rows,
                  int64_t row_bytes, int cols, int nslices, int rows_per_wg, int nw) {
    const int64_t row_begin = (int64_t)blockIdx.x * rows_per_wg;
    const int64_t row_end = row_begin + rows_per_wg < rows ? row_begin + rows_per_wg : rows;
    half_rows<FMT, T, D>(W, row_bytes, cols, nslices, x, row_begin, row_end, nw,
                         [=](int t, int64_t row, float v) { y[t * rows + row] = v; });
}

template <int FMT, int T, int R, int H>
__global__ void __launch_bounds__(64 * kMaxWaves)
qgemv_mx_kernel(const uint8_t* __restrict__ W, const float* __restrict__ x, float* __restrict__ y, int64_t rows,
                int64_t row_bytes, int cols, int nslices, int rows_per_wg, int nw) {
    const int64_t row_begin = (int64_t)blockIdx.x * rows_per_wg;
    const int64_t row_end = row_begin + rows_per_wg < rows ? row_begin + rows_per_wg : rows;
    int64_t xoff[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xoff[t] = (int64_t)t * cols;
    float4 xv[T][H];
    mx_load_x<FMT, T, H>(x, xoff, nslices, xv);
    mx_rows<FMT, T, R, false, H, false, kDensePolicy<FMT>>(W, row_bytes, nslices, xv, row_begin, row_end, nw,
                    [=](int t, int64_t row, float v) { y[t * rows + row] = v; });
}

template <int FMT, int T, int D>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_units_kernel(DenseArgs a) {
    const int64_t row_begin = (int64_t)blockIdx.x * a.rows_per_wg;
    const int64_t row_end = row_begin + a.rows_per_wg < a.rows ? row_begin + a.rows_per_wg : a.rows;
    float* __restrict__ y = a.y;
    const int64_t rows = a.rows;
    unit_rows<FMT, T, D>(a.W, a.row_bytes, a.cols, a.nslices, a.x, row_begin, row_end,
                         [=](int t, int64_t row, float v) { y[t * rows + row] = v; });
}

template <int T>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_mfma_persist_kernel(DenseArgs a) {
    int64_t xoff[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xoff[t] = (int64_t)t * a.cols;
    float* __restrict__ y = a.y;
    const int64_t rows = a.rows;
    mfma_persist_q8<T>(a.W, a.rows, a.row_bytes, a.cols, a.nslices, a.rows_per_wg / 16, a.x, xoff,
                       [=](int t, int64_t row, float v) { y[t * rows + row] = v; });
}

template <int FMT, int T, int ST, int D, bool XSEP>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_dma_argmax_kernel(DenseArgs a, unsigned long long* work) {
    const int64_t row_begin = (int64_t)blockIdx.x * a.rows_per_wg;
    const int64_t row_end = row_begin + a.rows_per_wg < a.rows ? row_begin + a.rows_per_wg : a.rows;
    int64_t xoff[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xoff[t] = (int64_t)t * a.cols;
    ArgmaxOut<T> best;
    dma_rows<FMT, T, ST, D, XSEP>(a.W, a.row_bytes, a.cols, a.nslices, a.x, xoff, row_begin, row_end,
                                  (int)(blockDim.x >> 6), best);
    best.merge(work);
}

template <int FMT, int T, int D>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_half_argmax_kernel(DenseArgs a, unsigned long long* work) {
    const int64_t row_begin = (int64_t)blockIdx.x * a.rows_per_wg;
    const int64_t row_end = row_begin + a.rows_per_wg < a.rows ? row_begin + a.rows_per_wg : a.rows;
    ArgmaxOut<T> best;
    half_rows<FMT, T, D>(a.W, a.row_bytes, a.cols, a.nslices, a.x, row_begin, row_end, (int)(blockDim.x >> 6), best);
    best.merge(work);
}

template <int FMT, int T>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_mxp_kernel(DenseArgs a) {
    float* __restrict__ y = a.y;
    const int64_t rows = a.rows;
    if (a.ybuf_rows == 0) {
        mxp_rows<FMT, T>(a.W, a.rows, a.row_bytes, a.cols, a.nslices, a.rows_per_wg / 16, a.x,
                         [=](int t, int64_t row, float v) { y[t * rows + row] = v; });
        return;
    }
    // The outputs wait in LDS and leave at the end as one contiguous run per token:
    // a chunk's 192-byte pieces of y, written as the chunks are summed, slowed the
    // weight stream they cut into by 2 µs at T = 1 and 9 µs at T = 4 on the LM head.
    using M = MxpShape<FMT>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int C = a.rows_per_wg / 16, nsl = a.nslices, cap = a.ybuf_rows;
    float* ybuf = reinterpret_cast<float*>(smem + (size_t)nsl * M::kSlot +
                                           (size_t)2 * C * nsl * 16 * pad_pow2(T) * 4 + 16);  // [T][cap]
    const int64_t TT = (rows + 15) / 16;
    const int64_t t0 = (int64_t)blockIdx.x * TT / gridDim.x, t1 = (int64_t)(blockIdx.x + 1) * TT / gridDim.x;
    const int64_t row_begin = t0 * 16;
    const int nr = (int)((t1 * 16 < rows ? t1 * 16 : rows) - row_begin);  // <= cap
    mxp_rows<FMT, T>(a.W, a.rows, a.row_bytes, a.cols, nsl, C, a.x,
                     [=](int t, int64_t row, float v) { ybuf[t * cap + (int)(row - row_begin)] = v; });
    __syncthreads();  // every chunk is summed
    for (int i = threadIdx.x; i < T * nr; i += blockDim.x) {
        const int t = i / nr, r = i - t * nr;
        y[t * rows + row_begin + r] = ybuf[t * cap + r];
    }
}

template <int FMT, int T>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_mxp_argmax_kernel(DenseArgs a, unsigned long long* work) {
    ArgmaxOut<T> best;
    mxp_rows<FMT, T>(a.W, a.rows, a.row_bytes, a.cols, a.nslices, a.rows_per_wg / 16, a.x, best);
    best.merge(work);
}

template <int FMT, int T, int R, int H>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_mx_argmax_kernel(DenseArgs a, unsigned long long* work) {
    const int64_t row_begin = (int64_t)blockIdx.x * a.rows_per_wg;
    const int64_t row_end = row_begin + a.rows_per_wg < a.rows ? row_begin + a.rows_per_wg : a.rows;
    ArgmaxOut<T> best;
    int64_t xoff[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xoff[t] = (int64_t)t * a.cols;
    float4 xv[T][H];
    mx_load_x<FMT, T, H>(a.x, xoff, a.nslices, xv);
    mx_rows<FMT, T, R, false, H, false, kDensePolicy<FMT>>(a.W, a.row_bytes, a.nslices, xv, row_begin, row_end,
                                                          (int)(blockDim.x >> 6), best);
    best.merge(work);
}

template <int T>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_persist_argmax_kernel(DenseArgs a, unsigned long long* work) {
    int64_t xoff[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xoff[t] = (int64_t)t * a.cols;
    ArgmaxOut<T> best;
    mfma_persist_q8<T>(a.W, a.rows, a.row_bytes, a.cols, a.nslices, a.rows_per_wg / 16, a.x, xoff, best);
    best.merge(work);
}

template <int FMT, int T, bool ONE_SHOT>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_dense_argmax_kernel(DenseArgs a, unsigned long long* work) {
    const int64_t row_begin = (int64_t)blockIdx.x * a.rows_per_wg;
    const int64_t row_end = row_begin + a.rows_per_wg < a.rows ? row_begin + a.rows_per_wg : a.rows;
    int64_t xoff[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xoff[t] = (int64_t)t * a.cols;
    ArgmaxOut<T> best;
    gemv_rows<FMT, T, 2, ONE_SHOT>(a.W, a.row_bytes, a.cols, a.nslices, a.x, xoff, row_begin, row_end,
                                   (int)(blockDim.x >> 6), best);
    best.merge(work);
}

template <int FMT, int T>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_stream_argmax_kernel(DenseArgs a, unsigned long long* work) {
    const int64_t row_begin = (int64_t)blockIdx.x * a.rows_per_wg;
    const int64_t row_end = row_begin + a.rows_per_wg < a.rows ? row_begin + a.rows_per_wg : a.rows;
    int64_t xoff[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xoff[t] = (int64_t)t * a.cols;
    ArgmaxOut<T> best;
    stream_rows<FMT, T, 8>(a.W, a.row_bytes, a.cols, a.nslices, a.x, xoff, row_begin, row_end, (int)(blockDim.x >> 6),
                           best);
    best.merge(work);
}

template <int FMT, int T>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_gather_kernel(DenseArgs a, const int32_t* ids, int64_t nsel) {
    const int64_t sel_begin = (int64_t)blockIdx.x * a.rows_per_wg;
    const int64_t sel_end = sel_begin + a.rows_per_wg < nsel ? sel_begin + a.rows_per_wg : nsel;
    float* __restrict__ y = a.y;
    gather_rows<FMT, T, 2>(a.W, a.rows, a.row_bytes, a.cols, a.nslices, ids, a.x, sel_begin, sel_end,
                           [=](int t, int64_t i, float v) { y[t * nsel + i] = v; });
}

// The row subset on the matrix cores: kind 8 (H = 1) or kind 11 (H = 2) over the ids
// of the workgroup's range, so y[t][i] is the dense call's y[t][ids[i]] of that kind.
template <int FMT, int T, int H>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_mx_gather_kernel(DenseArgs a, const int32_t* ids, int64_t nsel) {
    const int64_t sel_begin = (int64_t)blockIdx.x * a.rows_per_wg;
    const int64_t sel_end = sel_begin + a.rows_per_wg < nsel ? sel_begin + a.rows_per_wg : nsel;
    int64_t xoff[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xoff[t] = (int64_t)t * a.cols;
    float4 xv[T][H];
    mx_load_x<FMT, T, H>(a.x, xoff, a.nslices, xv);
    float* __restrict__ y = a.y;
    const int64_t rows = a.rows;
    mx_rows<FMT, T, 1, false, H, true>(
        a.W, a.row_bytes, a.nslices, xv, sel_begin, sel_end, (int)(blockDim.x >> 6),
        [=](int t, int64_t i, float v) {
            const int id = ids[i];
            y[t * nsel + i] = id >= 0 && id < rows ? v : __builtin_nanf("");
        },
        ids, rows);
}

template <int T>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_mfma_q8_kernel(DenseArgs a) {
    const int64_t row_begin = (int64_t)blockIdx.x * a.rows_per_wg;
    const int64_t row_end = row_begin + a.rows_per_wg < a.rows ? row_begin + a.rows_per_wg : a.rows;
    int64_t xoff[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xoff[t] = (int64_t)t * a.cols;
    float* __restrict__ y = a.y;
    const int64_t rows = a.rows;
    mfma_rows_q8<T>(a.W, a.row_bytes, a.cols, a.nslices, a.x, xoff, row_begin, row_end,
                    [=](int t, int64_t row, float v) { y[t * rows + row] = v; });
}

// Grouped experts: workgroup (slot, part, tile) with slot = (t, j).  Each
// expert's rows are streamed once for every token that chose it (the M5
// audit's expert grouping, section 1 item 2, done here inside each workgroup
// from the tiny ids array instead of a separate plan pass): the n workgroups
// whose slots name expert e split each tile of e's rows n ways, and each
// computes its share for all of e's tokens, so sharing costs no parallelism.
// Two parts: the gate and up tables of one expert in one launch (part 1 reads
// W2, writes y2).  Per-slot inputs (the down projection, whose input differs
// for every (token, expert) pair): the slots naming e form groups of up to T,
// each with its own x row, and the members of a group split its rows.

// The outputs a serving workgroup computes: ne activation vectors (tokens, or
// slots with per-slot inputs) and where each result goes.
struct GroupTargets {
    uint32_t tokmask;  // per-token inputs: bit t set = token t chose e
    uint64_t slots;    // up to 4 slot indices, 16 bits each: per-slot inputs, the group's slots;
                       // per-token inputs, the slot of each token (in token order) that names e
    int dup;           // per-token inputs: some token names e in more than one slot
    int ne;
    int rank, nwork;   // this workgroup's share of the rows: rank of nwork
};

// The share `rank` of `nwork` of a row range, in whole R-row tiles (possibly empty).
template <int R = 8>
__device__ __forceinline__ void share_rows(const GroupTargets& g, int64_t& row_begin, int64_t& row_end) {
    const int64_t nt = (row_end - row_begin + R - 1) / R;
    const int64_t t0 = nt * g.rank / g.nwork, t1 = nt * (g.rank + 1) / g.nwork;
    const int64_t e = row_begin + R * t1;
    row_begin += R * t0;
    if (e < row_end) row_end = e;
}

template <int NE>
__device__ __forceinline__ void group_offsets(const GroupedArgs& a, const GroupTargets& g, int64_t (&xoff)[NE]) {
    uint32_t m = g.tokmask;
#pragma unroll
    for (int n = 0; n < NE; ++n) {
        if (a.per_slot_x) {
            xoff[n] = (int64_t)((g.slots >> (16 * n)) & 0xFFFF) * a.cols;
        } else {
            xoff[n] = (int64_t)__builtin_ctz(m) * a.cols;
            m &= m - 1;
        }
    }
}

// Output n of a tile row: per-slot, its slot's row; per-token, every slot of the
// n-th token that names e (n varies across lanes, so no array indexing here).
__device__ __forceinline__ void group_store(const GroupedArgs& a, float* __restrict__ y, int e, const GroupTargets& g,
                                            int n, int64_t row, float v) {
    if (a.per_slot_x || !g.dup) {
        const int slot = (int)((g.slots >> (16 * n)) & 0xFFFF);
        y[(int64_t)slot * a.rows + row] = v;
        return;
    }
    uint32_t m = g.tokmask;
    for (int i = 0; i < n; ++i) m &= m - 1;
    const int t = __builtin_ctz(m);
    for (int j = 0; j < a.topk; ++j)
        if (a.ids[t * a.topk + j] == e) y[((int64_t)t * a.topk + j) * a.rows + row] = v;
}

template <int FMT, int NE, int RB, bool ONE_SHOT>
__device__ __forceinline__ void grouped_run(const GroupedArgs& a, const uint8_t* W, float* y, int e, const GroupTargets& g,
                                            int64_t row_begin, int64_t row_end) {
    int64_t xoff[NE];
    group_offsets<NE>(a, g, xoff);
    gemv_rows<FMT, NE, RB, ONE_SHOT>(W + (int64_t)e * a.expert_bytes, a.row_bytes, a.cols, a.nslices, a.x, xoff, row_begin,
                                     row_end, (int)(blockDim.x >> 6), [=](int n, int64_t row, float v) { group_store(a, y, e, g, n, row, v); });
}

// The slot, part and row range of a grouped workgroup and the expert it serves.
// Returns false when its id is out of range: its output rows are then NaN.
__device__ __forceinline__ bool grouped_slot(const GroupedArgs& a, int& e, const uint8_t*& W, float*& y,
                                             int64_t& row_begin, int64_t& row_end) {
    const int per_slot = a.tiles_per_expert * a.parts;
    const int slot = blockIdx.x / per_slot;
    int tile = blockIdx.x % per_slot;
    const int part = tile >= a.tiles_per_expert;
    tile -= part * a.tiles_per_expert;
    W = part ? a.W2 : a.W;
    y = part ? a.y2 : a.y;
    row_begin = (int64_t)tile * a.rows_per_wg;
    row_end = row_begin + a.rows_per_wg < a.rows ? row_begin + a.rows_per_wg : a.rows;
    e = a.ids[slot];
    if (e < 0 || e >= a.n_experts) {  // precondition violated: make it visible
        float* yrow = y + (int64_t)slot * a.rows;
        for (int64_t r = row_begin + threadIdx.x; r < row_end; r += blockDim.x) yrow[r] = __builtin_nanf("");
        return false;
    }
    return true;
}

// Bits of a 64-slot chunk starting at c that lie below `slot`.
__device__ __forceinline__ uint64_t below(int slot, int c) {
    return slot - c >= 64 ? ~0ull : slot - c <= 0 ? 0ull : (1ull << (slot - c)) - 1;
}

// Passes over ids, 64 at a time in parallel lanes: whom this workgroup computes
// for and its share of the rows.  Per-token inputs: every token that chose e;
// the workers are the slots naming e.  Per-slot inputs: the slots naming e in
// rank order form groups of T (one group when every token names an expert at
// most once); the workers are the group's slots.
// id0: the lane's id of the first 64 (-1 past the end), when loaded ahead.
__device__ __forceinline__ void grouped_targets(const GroupedArgs& a, int e, GroupTargets& g, int id0 = -2) {
    const int slot = blockIdx.x / (a.tiles_per_expert * a.parts);
    const int n = a.T * a.topk;
    const int lane = threadIdx.x & 63;
    g.tokmask = 0;
    g.slots = 0;
    g.dup = 0;
    g.ne = 0;
    int before = 0, total = 0;
    for (int c = 0; c < n; c += 64) {
        const int i = c + lane;
        const bool m = i < n && (c == 0 && id0 != -2 ? id0 : a.ids[i]) == e;
        const uint64_t b = __ballot(m);  // uniform
        before += __builtin_popcountll(b & below(slot, c));
        total += __builtin_popcountll(b);
        if (!a.per_slot_x) {
            // the slots naming e in ascending order: tokens come in ascending order,
            // so the k-th new token is the k-th of tokmask
            for (uint64_t bb = b; bb; bb &= bb - 1) {
                const int si = c + __builtin_ctzll(bb), t = si / a.topk;
                if (g.tokmask >> t & 1) {
                    g.dup = 1;
                } else {
                    g.slots |= (uint64_t)si << (16 * __builtin_popcount(g.tokmask));
                    g.tokmask |= 1u << t;
                }
            }
        }
    }
    if (!a.per_slot_x) {
        g.ne = __builtin_popcount(g.tokmask);
        g.rank = before;
        g.nwork = total;
        return;
    }
    const int G = a.T;  // inputs per group: at most T, what the workgroup's LDS is sized for
    const int g0 = before / G * G;
    g.rank = before - g0;
    g.nwork = total - g0 < G ? total - g0 : G;
    int rank = 0;  // rank of the first slot of the chunk among e's slots
    for (int c = 0; c < n && g.ne < g.nwork; c += 64) {
        const int i = c + lane;
        uint64_t b = __ballot(i < n && a.ids[i] == e);
        for (; b && g.ne < g.nwork; b &= b - 1, ++rank)
            if (rank >= g0) {
                g.slots |= (uint64_t)(c + __builtin_ctzll(b)) << (16 * g.ne);
                ++g.ne;
            }
    }
}

template <int FMT, int RB, bool ONE_SHOT>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_grouped_kernel(GroupedArgs a) {
    int e;
    const uint8_t* W;
    float* y;
    int64_t row_begin, row_end;
    GroupTargets g;
    if (!grouped_slot(a, e, W, y, row_begin, row_end)) return;
    grouped_targets(a, e, g);
    share_rows(g, row_begin, row_end);
    if (row_begin >= row_end) return;
    switch (g.ne) {
    case 1: grouped_run<FMT, 1, RB, ONE_SHOT>(a, W, y, e, g, row_begin, row_end); break;
    case 2: grouped_run<FMT, 2, RB, ONE_SHOT>(a, W, y, e, g, row_begin, row_end); break;
    case 3: grouped_run<FMT, 3, RB, ONE_SHOT>(a, W, y, e, g, row_begin, row_end); break;
    default: grouped_run<FMT, 4, RB, ONE_SHOT>(a, W, y, e, g, row_begin, row_end); break;
    }
}

// Grouped experts on the LDS-DMA streamed path (x staged apart, so any number of
// inputs per expert fits the same ring).
template <int FMT, int NE, int D, bool PRE>
__device__ __forceinline__ void grouped_dma_run(const GroupedArgs& a, const uint8_t* W, float* y, int e,
                                                const GroupTargets& g, int64_t row_begin, int64_t row_end) {
    int64_t xoff[NE];
    group_offsets<NE>(a, g, xoff);
    auto out = [=](int n, int64_t row, float v) { group_store(a, y, e, g, n, row, v); };
    dma_rows<FMT, NE, 8, D, true, decltype(out)&, PRE>(W + (int64_t)e * a.expert_bytes, a.row_bytes, a.cols, a.nslices,
                                                     a.x, xoff, row_begin, row_end, (int)(blockDim.x >> 6), out);
}

template <int FMT, int D, bool PRE>
__device__ __forceinline__ void grouped_dma_switch(const GroupedArgs& a, const uint8_t* W, float* y, int e,
                                                   const GroupTargets& g, int64_t row_begin, int64_t row_end) {
    switch (g.ne) {
    case 1: grouped_dma_run<FMT, 1, D, PRE>(a, W, y, e, g, row_begin, row_end); break;
    case 2: grouped_dma_run<FMT, 2, D, PRE>(a, W, y, e, g, row_begin, row_end); break;
    case 3: grouped_dma_run<FMT, 3, D, PRE>(a, W, y, e, g, row_begin, row_end); break;
    default: grouped_dma_run<FMT, 4, D, PRE>(a, W, y, e, g, row_begin, row_end); break;
    }
}

template <int FMT, int D>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_grouped_dma_kernel(GroupedArgs a) {
    int e;
    const uint8_t* W;
    float* y;
    int64_t row_begin, row_end;
    if (!grouped_slot(a, e, W, y, row_begin, row_end)) return;
    // the first tiles of the range start streaming while the ids are scanned;
    // they are this workgroup's own when its share starts the range
    dma_prefetch<FMT, 8, D>(W + (int64_t)e * a.expert_bytes, a.row_bytes, a.nslices, row_begin, row_end);
    GroupTargets g;
    grouped_targets(a, e, g);
    const int64_t first = row_begin;
    share_rows(g, row_begin, row_end);
    if (row_begin < row_end && row_begin == first) {
        grouped_dma_switch<FMT, D, true>(a, W, y, e, g, row_begin, row_end);
        return;
    }
    wait_vmcnt<0>();  // the prefetch is not this share's: drain it
    if (row_begin < row_end) grouped_dma_switch<FMT, D, false>(a, W, y, e, g, row_begin, row_end);
}

// Grouped experts on the matrix cores (kind 8's tiles): the same slots, sharing
// and outputs, the workgroup's rows shared in 16-row tiles; x of each input is
// split into its bf16 pieces per wave as on the dense path.
// Per-token inputs: every token's x of the wave's slice is loaded ahead (xall),
// and the group's NE inputs are picked from it; per-slot inputs are loaded here.
template <int FMT, int NE, int R, bool PRE>
__device__ __forceinline__ void grouped_mx_run(const GroupedArgs& a, const uint8_t* W, float* y, int e,
                                               const GroupTargets& g, const float4 (&xall)[QG_MAX_T],
                                               int64_t row_begin, int64_t row_end) {
    const int nsl = a.cols / kHalfSlice;
    float4 xv[NE][1];
    if (a.per_slot_x) {
        int64_t xoff[NE];
        group_offsets<NE>(a, g, xoff);
        mx_load_x<FMT, NE>(a.x, xoff, nsl, xv);
    } else {
        uint32_t m = g.tokmask;
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const int t = __builtin_ctz(m);  // uniform
            m &= m - 1;
#pragma unroll
            for (int u = 0; u < QG_MAX_T; ++u)
                if (u == t) xv[i][0] = xall[u];
        }
    }
    mx_rows<FMT, NE, R, PRE>(W + (int64_t)e * a.expert_bytes, a.row_bytes, nsl, xv, row_begin, row_end,
                             (int)(blockDim.x >> 6),
                             [=](int n, int64_t row, float v) { group_store(a, y, e, g, n, row, v); });
}

template <int FMT, int R, bool PRE>
__device__ __forceinline__ void grouped_mx_switch(const GroupedArgs& a, const uint8_t* W, float* y, int e,
                                                  const GroupTargets& g, const float4 (&xall)[QG_MAX_T],
                                                  int64_t row_begin, int64_t row_end) {
    switch (g.ne) {
    case 1: grouped_mx_run<FMT, 1, R, PRE>(a, W, y, e, g, xall, row_begin, row_end); break;
    case 2: grouped_mx_run<FMT, 2, R, PRE>(a, W, y, e, g, xall, row_begin, row_end); break;
    case 3: grouped_mx_run<FMT, 3, R, PRE>(a, W, y, e, g, xall, row_begin, row_end); break;
    default: grouped_mx_run<FMT, 4, R, PRE>(a, W, y, e, g, xall, row_begin, row_end); break;
    }
}

template <int FMT, int R>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_grouped_mx_kernel(GroupedArgs a) {
    // loads that do not depend on the expert go first: the first 64 ids of the
    // scan and (per-token inputs) every token's x; then the expert's first tile
    // starts streaming while the ids are scanned; it is this workgroup's own
    // when its share starts the range
    const int lane = threadIdx.x & 63;
    const int nid = a.T * a.topk;
    const int id0 = lane < nid ? a.ids[lane] : -1;
    float4 xall[QG_MAX_T];
    if (!a.per_slot_x) {
        const int k0 = ((int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) % (a.cols / kHalfSlice)) * kHalfSlice;
#pragma unroll
        for (int t = 0; t < QG_MAX_T; ++t)
            if (t < a.T) xall[t] = *reinterpret_cast<const float4*>(a.x + (int64_t)t * a.cols + k0 + 4 * lane);
    }
    int e;
    const uint8_t* W;
    float* y;
    int64_t row_begin, row_end;
    if (!grouped_slot(a, e, W, y, row_begin, row_end)) return;
    mx_prefetch<FMT, R>(W + (int64_t)e * a.expert_bytes, a.row_bytes, a.cols / kHalfSlice, row_begin, row_end);
    GroupTargets g;
    grouped_targets(a, e, g, id0);
    const int64_t first = row_begin;
    share_rows<16 * R>(g, row_begin, row_end);
    if (row_begin < row_end && row_begin == first) {
        grouped_mx_switch<FMT, R, true>(a, W, y, e, g, xall, row_begin, row_end);
        return;
    }
    wait_vmcnt<0>();  // the prefetch is not this share's: drain it
    if (row_begin < row_end) grouped_mx_switch<FMT, R, false>(a, W, y, e, g, xall, row_begin, row_end);
}

// --------------------------------------------------------------- dispatch
using DenseFn = void (*)(DenseArgs);
// the dense-path kernels with scalar arguments (W, x, y, rows, row_bytes, cols, nslices, rows_per_wg, nw)
using DmaFn = void (*)(const uint8_t*, const float*, float*, int64_t, int64_t, int, int, int, int);
using GroupedFn = void (*)(GroupedArgs);

int rb_index(int rb) { return rb == 1 ? 0 : rb == 2 ? 1 : rb == 4 ? 2 : rb == 8 ? 3 : 4; }

// Only the (format, T, RB, mode) combinations of the compiled set (tile_supported)
// are instantiated.
template <int FMT, int T, bool OS>
DmaFn dense_entry(int rbi) {
    constexpr int TP = pad_pow2(T);
    if (rbi == 0) return qgemv_dense_kernel<FMT, T, 1, OS>;
    if (rbi == 1) return qgemv_dense_kernel<FMT, T, 2, OS>;
    if constexpr (OS || T <= 3) {
        if (rbi == 2) return qgemv_dense_kernel<FMT, T, 4, OS>;
    }
    if constexpr ((OS && 8 * TP <= 32) || (!OS && T == 1 && FMT != QG_FMT_BF16)) {
        if (rbi == 3) return qgemv_dense_kernel<FMT, T, 8, OS>;
    }
    if constexpr (OS && 16 * TP <= 32) {
        if (rbi == 4) return qgemv_dense_kernel<FMT, T, 16, OS>;
    }
    return nullptr;
}

template <int FMT, bool OS>
DmaFn dense_for(int T, int rbi) {
    switch (T) {
    case 1: return dense_entry<FMT, 1, OS>(rbi);
    case 2: return dense_entry<FMT, 2, OS>(rbi);
    case 3: return dense_entry<FMT, 3, OS>(rbi);
    default: return dense_entry<FMT, 4, OS>(rbi);
    }
}

template <int FMT, bool OS>
GroupedFn grouped_for(int rbi) {
    // one kernel serves 1..4 tokens per expert, so it follows the T = 4 row of the set
    if (rbi == 0) return qgemv_grouped_kernel<FMT, 1, OS>;
    if (rbi == 1) return qgemv_grouped_kernel<FMT, 2, OS>;
    if constexpr (OS) {
        if (rbi == 2) return qgemv_grouped_kernel<FMT, 4, OS>;
        if (rbi == 3) return qgemv_grouped_kernel<FMT, 8, OS>;
    }
    return nullptr;
}

// the (format, T, tile) combinations of stream_supported: the ones that fit the
// register budget without spilling
template <int FMT, int T>
DmaFn stream_entry(int rb) {
    if constexpr (FMT != QG_FMT_BF16 || T <= 2) {
        if (rb == 4) return qgemv_stream_kernel<FMT, T, 8>;
    }
    if constexpr ((FMT == QG_FMT_Q8_0 && T == 1) || (FMT == QG_FMT_Q4_0 && T <= 2)) {
        if (rb == 8) return qgemv_stream_kernel<FMT, T, 16>;
    }
    return nullptr;
}

template <int FMT>
DmaFn stream_for(int T, int rb) {
    switch (T) {
    case 1: return stream_entry<FMT, 1>(rb);
    case 2: return stream_entry<FMT, 2>(rb);
    case 3: return stream_entry<FMT, 3>(rb);
    default: return stream_entry<FMT, 4>(rb);
    }
}

// LDS-DMA streamed kernels: 8-row tiles, ring depths 2, 3, 4, 6

template <int FMT, int T, int D>
DmaFn dma_depth(bool xsep) {
    if (xsep) return qgemv_dma_kernel<FMT, T, 8, D, true>;
    if constexpr (dma_x_slots<FMT, 8, T>() < D) return qgemv_dma_kernel<FMT, T, 8, D, false>;
    return nullptr;
}

template <int FMT, int T>
DmaFn dma_entry(int depth, bool xsep) {
    switch (depth) {
    case 2: return dma_depth<FMT, T, 2>(xsep);
    case 3: return dma_depth<FMT, T, 3>(xsep);
    case 4: return dma_depth<FMT, T, 4>(xsep);
    case 6: return dma_depth<FMT, T, 6>(xsep);
    default: return nullptr;
    }
}

template <int FMT>
DmaFn dma_for(int T, int depth, bool xsep) {
    switch (T) {
    case 1: return dma_entry<FMT, 1>(depth, xsep);
    case 2: return dma_entry<FMT, 2>(depth, xsep);
    case 3: return dma_entry<FMT, 3>(depth, xsep);
    default: return dma_entry<FMT, 4>(depth, xsep);
    }
}

template <int FMT, int T>
DenseFn units_entry(int depth) {
    switch (depth) {
    case 2: return qgemv_units_kernel<FMT, T, 2>;
    case 3: return qgemv_units_kernel<FMT, T, 3>;
    case 4: return qgemv_units_kernel<FMT, T, 4>;
    default: return nullptr;
    }
}

template <int FMT>
DenseFn units_for(int T, int depth) {
    switch (T) {
    case 1: return units_entry<FMT, 1>(depth);
    case 2: return units_entry<FMT, 2>(depth);
    case 3: return units_entry<FMT, 3>(depth);
    default: return units_entry<FMT, 4>(depth);
    }
}

template <int FMT>
DenseFn mfma_for(int T) {
    if constexpr (FMT == QG_FMT_Q8_0) {
        switch (T) {
        case 1: return qgemv_mfma_q8_kernel<1>;
        case 2: return qgemv_mfma_q8_kernel<2>;
        case 3: return qgemv_mfma_q8_kernel<3>;
        default: return qgemv_mfma_q8_kernel<4>;
        }
    }
    return nullptr;
}

}  // namespace

int launch_dense(int fmt, int T, const Tile& tile, const DenseArgs& a, void* stream) {
    const int rbi = rb_index(tile.rows_per_batch);
    DmaFn fn;
    if (one_shot(tile, a.nslices))
        fn = fmt == QG_FMT_Q8_0 ? dense_for<QG_FMT_Q8_0, true>(T, rbi)
           : fmt == QG_FMT_Q4_0 ? dense_for<QG_FMT_Q4_0, true>(T, rbi)
                                : dense_for<QG_FMT_BF16, true>(T, rbi);
    else
        fn = fmt == QG_FMT_Q8_0 ? dense_for<QG_FMT_Q8_0, false>(T, rbi)
           : fmt == QG_FMT_Q4_0 ? dense_for<QG_FMT_Q4_0, false>(T, rbi)
                                : dense_for<QG_FMT_BF16, false>(T, rbi);
    if (!fn) return (int)hipErrorInvalidValue;
    const int64_t nwg = (a.rows + tile.rows_per_wg - 1) / tile.rows_per_wg;
    hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(64 * tile.waves_per_wg), lds_bytes(tile, T), (hipStream_t)stream,
                       a.W, a.x, a.y, a.rows, a.row_bytes, a.cols, a.nslices, a.rows_per_wg, tile.waves_per_wg);
    return (int)hipGetLastError();
}

int launch_stream(int fmt, int T, const Tile& tile, const DenseArgs& a, void* stream) {
    DenseFn fn;
    if (tile.mfma == 2) {  // persistent: one workgroup per CU (at most one per 16-row tile)
        if (fmt != QG_FMT_Q8_0 || tile.rows_per_batch != 8 || tile.waves_per_wg != a.nslices) return (int)hipErrorInvalidValue;
        fn = T == 1 ? qgemv_mfma_persist_kernel<1> : T == 2 ? qgemv_mfma_persist_kernel<2>
           : T == 3 ? qgemv_mfma_persist_kernel<3> : qgemv_mfma_persist_kernel<4>;
        const int64_t tiles = (a.rows + 15) / 16;
        const int64_t nwg = tiles < kPersistGrid ? tiles : kPersistGrid;
        hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(64 * tile.waves_per_wg), mfma_persist_lds_bytes(tile, T),
                           (hipStream_t)stream, a);
        return (int)hipGetLastError();
    }
    const int64_t nwg = (a.rows + tile.rows_per_wg - 1) / tile.rows_per_wg;
    if (tile.mfma) {
        fn = tile.rows_per_batch != 8 ? nullptr
           : fmt == QG_FMT_Q8_0 ? mfma_for<QG_FMT_Q8_0>(T)
           : fmt == QG_FMT_Q4_0 ? mfma_for<QG_FMT_Q4_0>(T)
                                : mfma_for<QG_FMT_BF16>(T);
        if (!fn) return (int)hipErrorInvalidValue;
        hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(64 * tile.waves_per_wg),
                           stream_lds_bytes(fmt, tile, T, a.nslices), (hipStream_t)stream, a);
        return (int)hipGetLastError();
    }
    const DmaFn sfn = fmt == QG_FMT_Q8_0 ? stream_for<QG_FMT_Q8_0>(T, tile.rows_per_batch)
                    : fmt == QG_FMT_Q4_0 ? stream_for<QG_FMT_Q4_0>(T, tile.rows_per_batch)
                                         : stream_for<QG_FMT_BF16>(T, tile.rows_per_batch);
    if (!sfn) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(sfn, dim3((unsigned)nwg), dim3(64 * tile.waves_per_wg), stream_lds_bytes(fmt, tile, T, a.nslices),
                       (hipStream_t)stream, a.W, a.x, a.y, a.rows, a.row_bytes, a.cols, a.nslices, a.rows_per_wg,
                       tile.waves_per_wg);
    return (int)hipGetLastError();
}

int launch_dma(int fmt, int T, const Tile& tile, const DenseArgs& a, void* stream) {
    const bool xsep = tile.kind == 3;
    DmaFn fn = tile.rows_per_batch != 4 ? nullptr
             : fmt == QG_FMT_Q8_0 ? dma_for<QG_FMT_Q8_0>(T, tile.depth, xsep)
             : fmt == QG_FMT_Q4_0 ? dma_for<QG_FMT_Q4_0>(T, tile.depth, xsep)
                                  : dma_for<QG_FMT_BF16>(T, tile.depth, xsep);
    if (!fn) return (int)hipErrorInvalidValue;
    const int64_t nwg = (a.rows + tile.rows_per_wg - 1) / tile.rows_per_wg;
    hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(64 * tile.waves_per_wg), dma_lds_bytes(fmt, tile, T, a.nslices),
                       (hipStream_t)stream, a.W, a.x, a.y, a.rows, a.row_bytes, a.cols, a.nslices, a.rows_per_wg,
                       tile.waves_per_wg);
    return (int)hipGetLastError();
}

int launch_units(int fmt, int T, const Tile& tile, const DenseArgs& a, void* stream) {
    DenseFn fn = tile.rows_per_batch != 4 ? nullptr
               : fmt == QG_FMT_Q8_0 ? units_for<QG_FMT_Q8_0>(T, tile.depth)
               : fmt == QG_FMT_Q4_0 ? units_for<QG_FMT_Q4_0>(T, tile.depth)
                                    : units_for<QG_FMT_BF16>(T, tile.depth);
    if (!fn) return (int)hipErrorInvalidValue;
    const int64_t nwg = (a.rows + tile.rows_per_wg - 1) / tile.rows_per_wg;
    hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(64 * tile.waves_per_wg), units_lds_bytes(fmt, tile, T, a.cols),
                       (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

using ArgmaxFn = void (*)(DenseArgs, unsigned long long*);

template <int FMT, int T>
DmaFn half_entry(int depth) {
    switch (depth) {
    case 2: return qgemv_half_kernel<FMT, T, 2>;
    case 3: return qgemv_half_kernel<FMT, T, 3>;
    default: return nullptr;
    }
}

template <int FMT>
DmaFn half_for(int T, int depth) {
    switch (T) {
    case 1: return half_entry<FMT, 1>(depth);
    case 2: return half_entry<FMT, 2>(depth);
    case 3: return half_entry<FMT, 3>(depth);
    default: return half_entry<FMT, 4>(depth);
    }
}

template <int FMT, int T>
ArgmaxFn half_argmax_entry(int depth) {
    switch (depth) {
    case 2: return qgemv_half_argmax_kernel<FMT, T, 2>;
    case 3: return qgemv_half_argmax_kernel<FMT, T, 3>;
    default: return nullptr;
    }
}

template <int FMT>
ArgmaxFn half_argmax_for(int T, int depth) {
    switch (T) {
    case 1: return half_argmax_entry<FMT, 1>(depth);
    case 2: return half_argmax_entry<FMT, 2>(depth);
    case 3: return half_argmax_entry<FMT, 3>(depth);
    default: return half_argmax_entry<FMT, 4>(depth);
    }
}

template <int FMT, int R, int H>
DmaFn mx_entry(int T) {
    switch (T) {
    case 1: return qgemv_mx_kernel<FMT, 1, R, H>;
    case 2: return qgemv_mx_kernel<FMT, 2, R, H>;
    case 3: return qgemv_mx_kernel<FMT, 3, R, H>;
    default: return qgemv_mx_kernel<FMT, 4, R, H>;
    }
}

// R: 16-row groups per tile (1, 2); H: 256-wide halves per slice (1, 2; H = 2 with R = 1)
template <int FMT>
DmaFn mx_for(int T, int R, int H) {
    return H == 2 ? mx_entry<FMT, 1, 2>(T) : R == 2 ? mx_entry<FMT, 2, 1>(T) : mx_entry<FMT, 1, 1>(T);
}

template <int FMT, int R, int H>
ArgmaxFn mx_argmax_entry(int T) {
    switch (T) {
    case 1: return qgemv_mx_argmax_kernel<FMT, 1, R, H>;
    case 2: return qgemv_mx_argmax_kernel<FMT, 2, R, H>;
    case 3: return qgemv_mx_argmax_kernel<FMT, 3, R, H>;
    default: return qgemv_mx_argmax_kernel<FMT, 4, R, H>;
    }
}

template <int FMT>
ArgmaxFn mx_argmax_for(int T, int R, int H) {
    return H == 2 ? mx_argmax_entry<FMT, 1, 2>(T) : R == 2 ? mx_argmax_entry<FMT, 2, 1>(T) : mx_argmax_entry<FMT, 1, 1>(T);
}

template <int FMT>
DenseFn mxp_for(int T) {
    switch (T) {
    case 1: return qgemv_mxp_kernel<FMT, 1>;
    case 2: return qgemv_mxp_kernel<FMT, 2>;
    case 3: return qgemv_mxp_kernel<FMT, 3>;
    default: return qgemv_mxp_kernel<FMT, 4>;
    }
}

template <int FMT>
ArgmaxFn mxp_argmax_for(int T) {
    switch (T) {
    case 1: return qgemv_mxp_argmax_kernel<FMT, 1>;
    case 2: return qgemv_mxp_argmax_kernel<FMT, 2>;
    case 3: return qgemv_mxp_argmax_kernel<FMT, 3>;
    default: return qgemv_mxp_argmax_kernel<FMT, 4>;
    }
}

int launch_mxp(int fmt, int T, const Tile& tile, const DenseArgs& a_in, void* stream) {
    DenseArgs a = a_in;
    a.nslices = (int)(a.cols / kSlice);
    if (a.cols % kSlice || tile.waves_per_wg != a.nslices || tile.rows_per_wg % 16) return (int)hipErrorInvalidValue;
    const DenseFn fn = fmt == QG_FMT_Q8_0 ? mxp_for<QG_FMT_Q8_0>(T) : fmt == QG_FMT_Q4_0 ? mxp_for<QG_FMT_Q4_0>(T)
                                                                                      : mxp_for<QG_FMT_BF16>(T);
    const int64_t tiles = (a.rows + 15) / 16;
    const int64_t nwg = tiles < kPersistGrid ? tiles : kPersistGrid;
    // a workgroup's outputs stay in LDS when its (balanced) row range fits there
    size_t lds = mxp_lds_bytes(fmt, tile, T);
    const int64_t ycap = (tiles + nwg - 1) / nwg * 16;
    a.ybuf_rows = 0;
    const char* direct = getenv("QGEMV_P_DIRECT_STORES");
    if (!(direct && direct[0] == '1') && lds + mxp_ybuf_bytes(ycap, T) <= kMaxLds) {
        a.ybuf_rows = (int)ycap;
        lds += mxp_ybuf_bytes(ycap, T);
    }
    // one wave per 512-wide slice and one that sums the chunks
    hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(64 * (tile.waves_per_wg + 1)), lds, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

int launch_mx(int fmt, int T, const Tile& tile, const DenseArgs& a, void* stream) {
    const int H = tile.kind == 11 ? 2 : 1;
    const int nsl = (int)(a.cols / (kHalfSlice * H));
    if (a.cols % (kHalfSlice * H) || tile.waves_per_wg % nsl) return (int)hipErrorInvalidValue;
    const int R = tile.depth == 2 && H == 1 ? 2 : 1;
    const DmaFn fn = fmt == QG_FMT_Q8_0 ? mx_for<QG_FMT_Q8_0>(T, R, H) : fmt == QG_FMT_Q4_0 ? mx_for<QG_FMT_Q4_0>(T, R, H)
                                                                                           : mx_for<QG_FMT_BF16>(T, R, H);
    const int64_t nwg = (a.rows + tile.rows_per_wg - 1) / tile.rows_per_wg;
    hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(64 * tile.waves_per_wg), mx_lds_bytes(fmt, tile, T, nsl),
                       (hipStream_t)stream, a.W, a.x, a.y, a.rows, a.row_bytes, a.cols, nsl, a.rows_per_wg,
                       tile.waves_per_wg);
    return (int)hipGetLastError();
}

int launch_half(int fmt, int T, const Tile& tile, const DenseArgs& a, void* stream) {
    const int nsl = (int)(a.cols / kHalfSlice);
    if (tile.rows_per_batch != 4 || a.cols % kHalfSlice || tile.waves_per_wg % nsl) return (int)hipErrorInvalidValue;
    const DmaFn fn = fmt == QG_FMT_Q8_0 ? half_for<QG_FMT_Q8_0>(T, tile.depth)
                   : fmt == QG_FMT_Q4_0 ? half_for<QG_FMT_Q4_0>(T, tile.depth)
                                        : half_for<QG_FMT_BF16>(T, tile.depth);
    if (!fn) return (int)hipErrorInvalidValue;
    const int64_t nwg = (a.rows + tile.rows_per_wg - 1) / tile.rows_per_wg;
    hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(64 * tile.waves_per_wg), half_lds_bytes(fmt, tile, T, nsl),
                       (hipStream_t)stream, a.W, a.x, a.y, a.rows, a.row_bytes, a.cols, nsl, a.rows_per_wg,
                       tile.waves_per_wg);
    return (int)hipGetLastError();
}


template <int FMT, int T>
ArgmaxFn argmax_dma_entry(int depth, bool xsep) {
    auto pick = [&](auto dtag) -> ArgmaxFn {
        constexpr int D = decltype(dtag)::value;
        if (xsep) return qgemv_dma_argmax_kernel<FMT, T, 8, D, true>;
        if constexpr (dma_x_slots<FMT, 8, T>() < D) return qgemv_dma_argmax_kernel<FMT, T, 8, D, false>;
        return nullptr;
    };
    switch (depth) {
    case 2: return pick(std::integral_constant<int, 2>{});
    case 3: return pick(std::integral_constant<int, 3>{});
    case 4: return pick(std::integral_constant<int, 4>{});
    default: return nullptr;
    }
}

template <int FMT>
ArgmaxFn argmax_dma_for(int T, int depth, bool xsep) {
    switch (T) {
    case 1: return argmax_dma_entry<FMT, 1>(depth, xsep);
    case 2: return argmax_dma_entry<FMT, 2>(depth, xsep);
    case 3: return argmax_dma_entry<FMT, 3>(depth, xsep);
    default: return argmax_dma_entry<FMT, 4>(depth, xsep);
    }
}

template <int FMT>
ArgmaxFn argmax_stream_for(int T) {
    switch (T) {
    case 1: return qgemv_stream_argmax_kernel<FMT, 1>;
    case 2: return qgemv_stream_argmax_kernel<FMT, 2>;
    case 3:
        if constexpr (FMT != QG_FMT_BF16) return qgemv_stream_argmax_kernel<FMT, 3>;
        return nullptr;
    default:
        if constexpr (FMT != QG_FMT_BF16) return qgemv_stream_argmax_kernel<FMT, 4>;
        return nullptr;
    }
}

template <int FMT>
ArgmaxFn argmax_dense_for(int T, bool os) {
    switch (T) {
    case 1: return os ? qgemv_dense_argmax_kernel<FMT, 1, true> : qgemv_dense_argmax_kernel<FMT, 1, false>;
    case 2: return os ? qgemv_dense_argmax_kernel<FMT, 2, true> : qgemv_dense_argmax_kernel<FMT, 2, false>;
    case 3: return os ? qgemv_dense_argmax_kernel<FMT, 3, true> : qgemv_dense_argmax_kernel<FMT, 3, false>;
    default: return os ? qgemv_dense_argmax_kernel<FMT, 4, true> : qgemv_dense_argmax_kernel<FMT, 4, false>;
    }
}

int launch_argmax(int fmt, int T, const Tile& tile, const DenseArgs& a_in, void* work, int32_t* idx, float* val,
                  void* stream) {
    ArgmaxFn fn = nullptr;
    int64_t nwg = 0;
    size_t lds = 0;
    int waves = tile.waves_per_wg;
    DenseArgs a = a_in;
    if (tile.kind == 9 && a.cols % kSlice == 0 && tile.waves_per_wg == a.cols / kSlice && tile.rows_per_wg % 16 == 0) {
        a.nslices = a.cols / kSlice;
        fn = fmt == QG_FMT_Q8_0 ? mxp_argmax_for<QG_FMT_Q8_0>(T)
           : fmt == QG_FMT_Q4_0 ? mxp_argmax_for<QG_FMT_Q4_0>(T)
                                : mxp_argmax_for<QG_FMT_BF16>(T);
        const int64_t tiles = (a.rows + 15) / 16;
        nwg = tiles < kPersistGrid ? tiles : kPersistGrid;
        lds = mxp_lds_bytes(fmt, tile, T);
        waves = tile.waves_per_wg + 1;  // and the wave that sums the chunks
    } else if ((tile.kind == 8 || tile.kind == 11) && a.cols % (kHalfSlice * (tile.kind == 11 ? 2 : 1)) == 0 &&
               tile.waves_per_wg % (a.cols / (kHalfSlice * (tile.kind == 11 ? 2 : 1))) == 0) {
        const int H = tile.kind == 11 ? 2 : 1;
        a.nslices = a.cols / (kHalfSlice * H);  // 256- or 512-wide slices
        const int R = tile.depth == 2 && H == 1 ? 2 : 1;
        fn = fmt == QG_FMT_Q8_0 ? mx_argmax_for<QG_FMT_Q8_0>(T, R, H)
           : fmt == QG_FMT_Q4_0 ? mx_argmax_for<QG_FMT_Q4_0>(T, R, H)
                                : mx_argmax_for<QG_FMT_BF16>(T, R, H);
        nwg = (a.rows + tile.rows_per_wg - 1) / tile.rows_per_wg;
        lds = mx_lds_bytes(fmt, tile, T, a.nslices);
    } else if (tile.kind == 7 && tile.rows_per_batch == 4 && a.cols % kHalfSlice == 0 &&
        tile.waves_per_wg % (a.cols / kHalfSlice) == 0) {
        a.nslices = a.cols / kHalfSlice;  // 256-wide slices
        fn = fmt == QG_FMT_Q8_0 ? half_argmax_for<QG_FMT_Q8_0>(T, tile.depth)
           : fmt == QG_FMT_Q4_0 ? half_argmax_for<QG_FMT_Q4_0>(T, tile.depth)
                                : half_argmax_for<QG_FMT_BF16>(T, tile.depth);
        nwg = (a.rows + tile.rows_per_wg - 1) / tile.rows_per_wg;
        lds = half_lds_bytes(fmt, tile, T, a.nslices);
    } else if (tile.kind == 1 && tile.mfma == 2 && fmt == QG_FMT_Q8_0 && tile.rows_per_batch == 8 &&
        tile.waves_per_wg == a.nslices) {
        fn = T == 1 ? qgemv_persist_argmax_kernel<1> : T == 2 ? qgemv_persist_argmax_kernel<2>
           : T == 3 ? qgemv_persist_argmax_kernel<3> : qgemv_persist_argmax_kernel<4>;
        const int64_t tiles = (a.rows + 15) / 16;
        nwg = tiles < kPersistGrid ? tiles : kPersistGrid;
        lds = mfma_persist_lds_bytes(tile, T);
    } else if ((tile.kind == 2 || tile.kind == 3) && tile.rows_per_batch == 4) {
        const bool xsep = tile.kind == 3;
        fn = fmt == QG_FMT_Q8_0 ? argmax_dma_for<QG_FMT_Q8_0>(T, tile.depth, xsep)
           : fmt == QG_FMT_Q4_0 ? argmax_dma_for<QG_FMT_Q4_0>(T, tile.depth, xsep)
                                : argmax_dma_for<QG_FMT_BF16>(T, tile.depth, xsep);
        nwg = (a.rows + tile.rows_per_wg - 1) / tile.rows_per_wg;
        lds = dma_lds_bytes(fmt, tile, T, a.nslices);
    } else if (tile.kind == 1 && !tile.mfma && tile.rows_per_batch == 4 && stream_supported(fmt, T, 4)) {
        fn = fmt == QG_FMT_Q8_0 ? argmax_stream_for<QG_FMT_Q8_0>(T)
           : fmt == QG_FMT_Q4_0 ? argmax_stream_for<QG_FMT_Q4_0>(T)
                                : argmax_stream_for<QG_FMT_BF16>(T);
        nwg = (a.rows + tile.rows_per_wg - 1) / tile.rows_per_wg;
        lds = stream_lds_bytes(fmt, tile, T, a.nslices);
    } else if (tile.kind == 0 && tile.rows_per_batch == 2) {
        const bool os = one_shot(tile, a.nslices);
        fn = fmt == QG_FMT_Q8_0 ? argmax_dense_for<QG_FMT_Q8_0>(T, os)
           : fmt == QG_FMT_Q4_0 ? argmax_dense_for<QG_FMT_Q4_0>(T, os)
                                : argmax_dense_for<QG_FMT_BF16>(T, os);
        nwg = (a.rows + tile.rows_per_wg - 1) / tile.rows_per_wg;
        lds = lds_bytes(tile, T);
    }
    if (!fn) return (int)hipErrorInvalidValue;
    const size_t keys = (size_t)waves * T * 8;  // the workgroup merge's wave maxima
    if (lds < keys) lds = keys;
    unsigned long long* w = (unsigned long long*)work;
    hipLaunchKernelGGL(qgemv_argmax_init_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, w, T);
    hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(64 * waves), lds, (hipStream_t)stream, a, w);
    hipLaunchKernelGGL(qgemv_argmax_finish_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, (const unsigned long long*)w,
                       idx, val, T);
    return (int)hipGetLastError();
}

int launch_gather(int fmt, int T, const Tile& tile, const DenseArgs& a_in, const int32_t* ids, int64_t nsel, void* stream) {
    using GatherFn = void (*)(DenseArgs, const int32_t*, int64_t);
    GatherFn fn = nullptr;
    if (tile.kind == 8 || tile.kind == 11) {  // matrix cores on 256- or 512-wide slices
        DenseArgs a = a_in;
        const int H = tile.kind == 11 ? 2 : 1;
        a.nslices = (int)(a.cols / (kHalfSlice * H));
        if (a.cols % (kHalfSlice * H) || tile.waves_per_wg % a.nslices || tile.rows_per_wg > 128 ||
            tile.rows_per_wg % 16)
            return (int)hipErrorInvalidValue;
        auto pick = [&](auto ftag) -> GatherFn {
            constexpr int F = decltype(ftag)::value;
            if (H == 2) {
                switch (T) {
                case 1: return qgemv_mx_gather_kernel<F, 1, 2>;
                case 2: return qgemv_mx_gather_kernel<F, 2, 2>;
                case 3: return qgemv_mx_gather_kernel<F, 3, 2>;
                default: return qgemv_mx_gather_kernel<F, 4, 2>;
                }
            }
            switch (T) {
            case 1: return qgemv_mx_gather_kernel<F, 1, 1>;
            case 2: return qgemv_mx_gather_kernel<F, 2, 1>;
            case 3: return qgemv_mx_gather_kernel<F, 3, 1>;
            default: return qgemv_mx_gather_kernel<F, 4, 1>;
            }
        };
        fn = fmt == QG_FMT_Q8_0 ? pick(std::integral_constant<int, QG_FMT_Q8_0>{})
           : fmt == QG_FMT_Q4_0 ? pick(std::integral_constant<int, QG_FMT_Q4_0>{})
                                : pick(std::integral_constant<int, QG_FMT_BF16>{});
        const int64_t nwg = (nsel + tile.rows_per_wg - 1) / tile.rows_per_wg;
        hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(64 * tile.waves_per_wg), mx_lds_bytes(fmt, tile, T, a.nslices),
                           (hipStream_t)stream, a, ids, nsel);
        return (int)hipGetLastError();
    }
    const DenseArgs& a = a_in;
    auto pick = [&](auto ftag) -> GatherFn {
        constexpr int F = decltype(ftag)::value;
        switch (T) {
        case 1: return qgemv_gather_kernel<F, 1>;
        case 2: return qgemv_gather_kernel<F, 2>;
        case 3: return qgemv_gather_kernel<F, 3>;
        default: return qgemv_gather_kernel<F, 4>;
        }
    };
    fn = fmt == QG_FMT_Q8_0 ? pick(std::integral_constant<int, QG_FMT_Q8_0>{})
       : fmt == QG_FMT_Q4_0 ? pick(std::integral_constant<int, QG_FMT_Q4_0>{})
                            : pick(std::integral_constant<int, QG_FMT_BF16>{});
    const int64_t nwg = (nsel + tile.rows_per_wg - 1) / tile.rows_per_wg;
    hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(64 * tile.waves_per_wg), gather_lds_bytes(fmt, tile, T, a.nslices),
                       (hipStream_t)stream, a, ids, nsel);
    return (int)hipGetLastError();
}

int launch_grouped(int fmt, const Tile& tile, const GroupedArgs& a, void* stream) {
    if (tile.kind == 8) {
        const int nsl = a.cols / kHalfSlice;
        if (a.cols % kHalfSlice || tile.waves_per_wg % nsl || tile.rows_per_wg % 16) return (int)hipErrorInvalidValue;
        const bool r2 = tile.depth == 2;
        const GroupedFn fn = fmt == QG_FMT_Q8_0 ? (r2 ? qgemv_grouped_mx_kernel<QG_FMT_Q8_0, 2> : qgemv_grouped_mx_kernel<QG_FMT_Q8_0, 1>)
                           : fmt == QG_FMT_Q4_0 ? (r2 ? qgemv_grouped_mx_kernel<QG_FMT_Q4_0, 2> : qgemv_grouped_mx_kernel<QG_FMT_Q4_0, 1>)
                                                : (r2 ? qgemv_grouped_mx_kernel<QG_FMT_BF16, 2> : qgemv_grouped_mx_kernel<QG_FMT_BF16, 1>);
        const int64_t nwg = (int64_t)a.T * a.topk * a.tiles_per_expert * a.parts;
        hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(64 * tile.waves_per_wg), mx_lds_bytes(fmt, tile, a.T, nsl),
                           (hipStream_t)stream, a);
        return (int)hipGetLastError();
    }
    if (tile.kind == 3) {
        GroupedFn fn = nullptr;
        if (tile.rows_per_batch == 4 && tile.depth == 2)
            fn = fmt == QG_FMT_Q8_0 ? qgemv_grouped_dma_kernel<QG_FMT_Q8_0, 2>
               : fmt == QG_FMT_Q4_0 ? qgemv_grouped_dma_kernel<QG_FMT_Q4_0, 2>
                                    : qgemv_grouped_dma_kernel<QG_FMT_BF16, 2>;
        if (tile.rows_per_batch == 4 && tile.depth == 3)
            fn = fmt == QG_FMT_Q8_0 ? qgemv_grouped_dma_kernel<QG_FMT_Q8_0, 3>
               : fmt == QG_FMT_Q4_0 ? qgemv_grouped_dma_kernel<QG_FMT_Q4_0, 3>
                                    : qgemv_grouped_dma_kernel<QG_FMT_BF16, 3>;
        if (!fn) return (int)hipErrorInvalidValue;
        const int64_t nwg = (int64_t)a.T * a.topk * a.tiles_per_expert * a.parts;
        hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(64 * tile.waves_per_wg), dma_lds_bytes(fmt, tile, a.T, a.nslices),
                           (hipStream_t)stream, a);
        return (int)hipGetLastError();
    }
    const int rbi = rb_index(tile.rows_per_batch);
    GroupedFn fn;
    if (one_shot(tile, a.nslices))
        fn = fmt == QG_FMT_Q8_0 ? grouped_for<QG_FMT_Q8_0, true>(rbi)
           : fmt == QG_FMT_Q4_0 ? grouped_for<QG_FMT_Q4_0, true>(rbi)
                                : grouped_for<QG_FMT_BF16, true>(rbi);
    else
        fn = fmt == QG_FMT_Q8_0 ? grouped_for<QG_FMT_Q8_0, false>(rbi)
           : fmt == QG_FMT_Q4_0 ? grouped_for<QG_FMT_Q4_0, false>(rbi)
                                : grouped_for<QG_FMT_BF16, false>(rbi);
    if (!fn) return (int)hipErrorInvalidValue;
    const int64_t nwg = (int64_t)a.T * a.topk * a.tiles_per_expert * a.parts;
    hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(64 * tile.waves_per_wg), lds_bytes(tile, a.T), (hipStream_t)stream,
                       a);
    return (int)hipGetLastError();
}

const char* hip_error_name(int err) { return hipGetErrorString((hipError_t)err); }

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int argmax_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {  // once per device, with that device current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        if (!p) return (int)hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return 0;
}

}  // namespace qg
