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
#include <stdint.h>

#include "qgemv_internal.h"

namespace qg {
namespace {

struct __attribute__((packed, aligned(2))) U4u { uint32_t v[4]; };  // 16 B at 2-byte alignment
struct __attribute__((packed, aligned(2))) U2u { uint32_t v[2]; };  // 8 B at 2-byte alignment
struct __attribute__((aligned(16))) U4a { uint32_t v[4]; };

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// ---------------------------------------------------------------- formats
// Each format says which k positions lane li owns inside a 512-wide slice, how
// to fetch the lane's bytes for one row, and how to turn them into 16 fp32
// weights (up to a per-block scale).
template <int FMT> struct Fmt;

template <> struct Fmt<QG_FMT_Q8_0> {
    static constexpr int kBlockBytes = 34;
    static constexpr bool kScaled = true;
    struct Raw { uint32_t c[4]; uint32_t d; };
    // block q = li / 2 of the slice, codes [16 h, 16 h + 16) with h = li % 2
    __device__ static int kpos(int li, int i) { return 32 * (li >> 1) + 16 * (li & 1) + i; }
    __device__ static int64_t slice_offset(int s) { return (int64_t)s * 16 * kBlockBytes; }
    __device__ static bool lane_valid(int li, int kslice0, int cols) { return kslice0 + 32 * (li >> 1) < cols; }
    __device__ static Raw load(const uint8_t* slice, int li) {
        const uint8_t* blk = slice + (li >> 1) * kBlockBytes;
        const U4u q = *reinterpret_cast<const U4u*>(blk + 2 + 16 * (li & 1));
        Raw r;
        r.c[0] = q.v[0]; r.c[1] = q.v[1]; r.c[2] = q.v[2]; r.c[3] = q.v[3];
        r.d = *reinterpret_cast<const uint16_t*>(blk);
        return r;
    }
    __device__ static Raw zero() { Raw r; r.c[0] = r.c[1] = r.c[2] = r.c[3] = 0; r.d = 0; return r; }
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
    // codes 8h .. 8h+7 (i < 8), high nibbles codes 16 + 8h .. 16 + 8h + 7 (i >= 8)
    __device__ static int kpos(int li, int i) {
        return 32 * (li >> 1) + (i < 8 ? 8 * (li & 1) + i : 16 + 8 * (li & 1) + (i - 8));
    }
    __device__ static int64_t slice_offset(int s) { return (int64_t)s * 16 * kBlockBytes; }
    __device__ static bool lane_valid(int li, int kslice0, int cols) { return kslice0 + 32 * (li >> 1) < cols; }
    __device__ static Raw load(const uint8_t* slice, int li) {
        const uint8_t* blk = slice + (li >> 1) * kBlockBytes;
        const U2u q = *reinterpret_cast<const U2u*>(blk + 2 + 8 * (li & 1));
        Raw r;
        r.c[0] = q.v[0]; r.c[1] = q.v[1];
        r.d = *reinterpret_cast<const uint16_t*>(blk);
        return r;
    }
    __device__ static Raw zero() { Raw r; r.c[0] = r.c[1] = 0; r.d = 0; return r; }
    // codes are returned as 16 * (c - 8): flipping bit 3 of a nibble gives the
    // 4-bit two's complement of c - 8, and shifting it to the top of a byte makes
    // a signed byte; the 16 is taken back out of the scale (exact: a power of 2).
    __device__ static float scale(const Raw& r) { return half_bits_to_float(r.d) * 0.0625f; }
    __device__ static float weight(const Raw& r, int i) {
        const uint32_t w = r.c[(i & 7) >> 2] ^ 0x88888888u;
        const uint32_t b = (i < 8) ? (w << 4) : w;  // nibble to the top of its byte
        return (float)(int32_t)(int8_t)((b >> (8 * (i & 3) + 0)) & 0xF0u);
    }
};

template <> struct Fmt<QG_FMT_BF16> {
    static constexpr bool kScaled = false;
    struct Raw { uint32_t c[8]; };
    // values [16 li, 16 li + 16) of the slice
    __device__ static int kpos(int li, int i) { return 16 * li + i; }
    __device__ static int64_t slice_offset(int s) { return (int64_t)s * kSlice * 2; }
    __device__ static bool lane_valid(int li, int kslice0, int cols) { return kslice0 + 16 * li < cols; }
    __device__ static Raw load_masked(const uint8_t* slice, int li, int kslice0, int cols) {
        const U4a* p = reinterpret_cast<const U4a*>(slice + 32 * li);
        const U4a a = p[0];
        Raw r;
        r.c[0] = a.v[0]; r.c[1] = a.v[1]; r.c[2] = a.v[2]; r.c[3] = a.v[3];
        if (kslice0 + 16 * li + 8 < cols) {
            const U4a b = p[1];
            r.c[4] = b.v[0]; r.c[5] = b.v[1]; r.c[6] = b.v[2]; r.c[7] = b.v[3];
        } else {
            r.c[4] = r.c[5] = r.c[6] = r.c[7] = 0;
        }
        return r;
    }
    __device__ static Raw zero() { Raw r; for (int i = 0; i < 8; ++i) r.c[i] = 0; return r; }
    __device__ static float scale(const Raw&) { return 1.0f; }
    __device__ static float weight(const Raw& r, int i) {
        const uint32_t w = r.c[i >> 1];
        return __builtin_bit_cast(float, (i & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
};

template <int FMT>
__device__ __forceinline__ typename Fmt<FMT>::Raw load_lane(const uint8_t* slice, int li, int kslice0, int cols,
                                                            bool row_ok) {
    using F = Fmt<FMT>;
    if (!row_ok || !F::lane_valid(li, kslice0, cols)) return F::zero();
    if constexpr (FMT == QG_FMT_BF16) return F::load_masked(slice, li, kslice0, cols);
    else return F::load(slice, li);
}

// ------------------------------------------------------------- reduction
// Halving butterfly over the 32 lanes of a row: with N values per lane, stage m
// (16, 8, 4, 2, 1) pairs lane li with li ^ m; the lane with bit m set keeps the
// upper half of its values and adds its partner's upper half, the other keeps
// the lower half.  After 5 stages value v's sum over all 32 lanes sits in the
// lanes whose index() is v.  The pairing of lanes at each stage -- hence every
// value's addition tree -- does not depend on N.
template <int N>
__device__ __forceinline__ void butterfly32(float (&v)[N], int li) {
#pragma unroll
    for (int st = 0; st < 5; ++st) {
        const int m = 16 >> st;
        const int cnt = N >> st;
        if (cnt >= 2) {
            const bool up = (li & m) != 0;
#pragma unroll
            for (int i = 0; i < cnt / 2; ++i) {
                const float send = up ? v[i] : v[i + cnt / 2];
                const float keep = up ? v[i + cnt / 2] : v[i];
                v[i] = keep + __shfl_xor(send, m, 64);
            }
        } else {
            v[0] = v[0] + __shfl_xor(v[0], m, 64);
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
// Cross-wave reduction without barriers: every batch of 2*RB rows has its own
// LDS slots [wave][row group][value] and an arrival counter.  A wave writes its
// butterfly results, then bumps the counter; the wave that arrives last adds the
// NW partial sets in wave order and stores the outputs.  No wave ever waits for
// another, and no slot is reused within a launch.
template <int FMT, int NT, int RB, class Out>
__device__ __forceinline__ void gemv_rows(const uint8_t* __restrict__ W, int64_t row_bytes, int cols, int nslices,
                                          const float* __restrict__ x, const int64_t (&xoff)[NT], int64_t row_begin,
                                          int64_t row_end, Out out) {
    using F = Fmt<FMT>;
    constexpr int TP = pad_pow2(NT);
    constexpr int N = RB * TP;  // values per lane entering the butterfly
    static_assert(N <= 32, "rows_per_batch * tokens too large");
    extern __shared__ float lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nw = blockDim.x >> 6;
    const int g = lane >> 5;   // which of the two rows of a step
    const int li = lane & 31;  // lane within the row
    const int nbatch = (int)((row_end - row_begin + 2 * RB - 1) / (2 * RB));
    float* part = lds;                                             // [nbatch][nw][2][N]
    int* arrivals = reinterpret_cast<int*>(lds + (size_t)nbatch * nw * 2 * N);  // [nbatch]
    for (int i = tid; i < nbatch; i += blockDim.x) arrivals[i] = 0;
    __syncthreads();

    bool writer;
    const int my_idx = butterfly_index<N>(li, writer);

    float xr[NT][kWeightsPerLane];
    int loaded_slice = -1;

    for (int b = 0; b < nbatch; ++b) {
        const int64_t rb0 = row_begin + (int64_t)b * 2 * RB;
        float acc[RB][TP];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int t = 0; t < TP; ++t) acc[r][t] = 0.0f;

        for (int s = wave; s < nslices; s += nw) {
            const int k0 = s * kSlice;
            if (s != loaded_slice) {
                const bool ok = F::lane_valid(li, k0, cols);
#pragma unroll
                for (int n = 0; n < NT; ++n)
#pragma unroll
                    for (int i = 0; i < kWeightsPerLane; ++i) {
                        const int k = k0 + F::kpos(li, i);
                        xr[n][i] = (ok && k < cols) ? x[xoff[n] + k] : 0.0f;
                    }
                loaded_slice = s;
            }
            typename F::Raw raw[RB];
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int64_t row = rb0 + 2 * r + g;
                const bool row_ok = row < row_end;
                raw[r] = load_lane<FMT>(W + (row_ok ? row : row_begin) * row_bytes + F::slice_offset(s), li, k0, cols,
                                        row_ok);
            }
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                float p[NT];
#pragma unroll
                for (int n = 0; n < NT; ++n) p[n] = 0.0f;
#pragma unroll
                for (int i = 0; i < kWeightsPerLane; ++i) {
                    const float w = F::weight(raw[r], i);
#pragma unroll
                    for (int n = 0; n < NT; ++n) p[n] = __builtin_fmaf(w, xr[n][i], p[n]);
                }
                if constexpr (F::kScaled) {
                    const float d = F::scale(raw[r]);
#pragma unroll
                    for (int n = 0; n < NT; ++n) acc[r][n] = __builtin_fmaf(d, p[n], acc[r][n]);
                } else {
#pragma unroll
                    for (int n = 0; n < NT; ++n) acc[r][n] = acc[r][n] + p[n];
                }
            }
        }

        float v[N];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int t = 0; t < TP; ++t) v[r * TP + t] = acc[r][t];
        butterfly32<N>(v, li);
        float* mine = part + (((size_t)b * nw + wave) * 2 + g) * N;
        if (writer) mine[my_idx] = v[0];
        // publish this wave's slots, then count the arrival (one atomic per wave)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        int prev = 0;
        if (lane == 0) prev = __hip_atomic_fetch_add(&arrivals[b], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
        prev = __shfl(prev, 0, 64);
        if (prev == nw - 1) {  // last arrival: all nw partial sets of batch b are in LDS
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
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
}

// ---------------------------------------------------------------- kernels
template <int FMT, int T, int RB>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_dense_kernel(DenseArgs a) {
    const int64_t row_begin = (int64_t)blockIdx.x * a.rows_per_wg;
    const int64_t row_end = row_begin + a.rows_per_wg < a.rows ? row_begin + a.rows_per_wg : a.rows;
    int64_t xoff[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xoff[t] = (int64_t)t * a.cols;
    float* __restrict__ y = a.y;
    const int64_t rows = a.rows;
    gemv_rows<FMT, T, RB>(a.W, a.row_bytes, a.cols, a.nslices, a.x, xoff, row_begin, row_end,
                          [=](int t, int64_t row, float v) { y[t * rows + row] = v; });
}

// Grouped experts: workgroup (slot, tile) with slot = (t, j).  The workgroup of
// the first slot that names expert e streams e's rows once for every token that
// chose e (the M5 audit's expert grouping, section 1 item 2, done here inside
// each workgroup from the tiny ids array instead of a separate plan pass);
// workgroups of later slots with the same e exit at once.
template <int FMT, int NE, int RB>
__device__ __forceinline__ void grouped_run(const GroupedArgs& a, int e, uint32_t tokmask, int64_t row_begin, int64_t row_end) {
    const uint32_t tokmask0 = tokmask;
    int tk[NE];  // the NE tokens that chose e, ascending
#pragma unroll
    for (int n = 0; n < NE; ++n) {
        tk[n] = __builtin_ctz(tokmask);
        tokmask &= tokmask - 1;
    }
    int64_t xoff[NE];
#pragma unroll
    for (int n = 0; n < NE; ++n) xoff[n] = (int64_t)tk[n] * a.cols;
    const int32_t* __restrict__ ids = a.ids;
    float* __restrict__ y = a.y;
    const int topk = a.topk;
    const int64_t rows = a.rows;
    gemv_rows<FMT, NE, RB>(a.W + (int64_t)e * a.expert_bytes, a.row_bytes, a.cols, a.nslices, a.x, xoff, row_begin,
                           row_end, [=](int n, int64_t row, float v) {
                               // token of output n: the n-th set bit of tokmask (n varies
                               // across lanes, so no array indexing here)
                               uint32_t m = tokmask0;
                               for (int i = 0; i < n; ++i) m &= m - 1;
                               const int t = __builtin_ctz(m);
                               for (int j = 0; j < topk; ++j)
                                   if (ids[t * topk + j] == e) y[((int64_t)t * topk + j) * rows + row] = v;
                           });
}

template <int FMT, int RB>
__global__ void __launch_bounds__(64 * kMaxWaves) qgemv_grouped_kernel(GroupedArgs a) {
    const int slot = blockIdx.x / a.tiles_per_expert;
    const int tile = blockIdx.x % a.tiles_per_expert;
    const int64_t row_begin = (int64_t)tile * a.rows_per_wg;
    const int64_t row_end = row_begin + a.rows_per_wg < a.rows ? row_begin + a.rows_per_wg : a.rows;
    const int e = a.ids[slot];
    if (e < 0 || e >= a.n_experts) {  // precondition violated: make it visible
        float* yrow = a.y + (int64_t)slot * a.rows;
        for (int64_t r = row_begin + threadIdx.x; r < row_end; r += blockDim.x) yrow[r] = __builtin_nanf("");
        return;
    }
    for (int i = 0; i < slot; ++i)
        if (a.ids[i] == e) return;  // an earlier slot's workgroup handles e
    uint32_t tokmask = 0;  // bit t: token t chose e
    for (int t = 0; t < a.T; ++t) {
        bool uses = false;
        for (int j = 0; j < a.topk; ++j) uses |= (a.ids[t * a.topk + j] == e);
        if (uses) tokmask |= 1u << t;
    }
    switch (__builtin_popcount(tokmask)) {
    case 1: grouped_run<FMT, 1, RB>(a, e, tokmask, row_begin, row_end); break;
    case 2: grouped_run<FMT, 2, RB>(a, e, tokmask, row_begin, row_end); break;
    case 3: grouped_run<FMT, 3, RB>(a, e, tokmask, row_begin, row_end); break;
    default: grouped_run<FMT, 4, RB>(a, e, tokmask, row_begin, row_end); break;
    }
}

// --------------------------------------------------------------- dispatch
using DenseFn = void (*)(DenseArgs);
using GroupedFn = void (*)(GroupedArgs);

int rb_index(int rb) { return rb == 1 ? 0 : rb == 2 ? 1 : rb == 4 ? 2 : 3; }

// Only the (T, RB) pairs of the compiled set (tile_supported) are instantiated.
template <int FMT, int T>
DenseFn dense_entry(int rbi) {
    if (rbi == 0) return qgemv_dense_kernel<FMT, T, 1>;
    if (rbi == 1) return qgemv_dense_kernel<FMT, T, 2>;
    if constexpr (T <= 3) {
        if (rbi == 2) return qgemv_dense_kernel<FMT, T, 4>;
    }
    if constexpr (T == 1) {
        if (rbi == 3) return qgemv_dense_kernel<FMT, T, 8>;
    }
    return nullptr;
}

template <int FMT>
DenseFn dense_for(int T, int rbi) {
    switch (T) {
    case 1: return dense_entry<FMT, 1>(rbi);
    case 2: return dense_entry<FMT, 2>(rbi);
    case 3: return dense_entry<FMT, 3>(rbi);
    default: return dense_entry<FMT, 4>(rbi);
    }
}

template <int FMT>
GroupedFn grouped_for(int rbi) {
    // one kernel serves 1..4 tokens per expert, so it takes the T = 4 limit on RB
    if (rbi == 0) return qgemv_grouped_kernel<FMT, 1>;
    if (rbi == 1) return qgemv_grouped_kernel<FMT, 2>;
    return nullptr;
}

}  // namespace

int launch_dense(int fmt, int T, const Tile& tile, const DenseArgs& a, void* stream) {
    const int rbi = rb_index(tile.rows_per_batch);
    DenseFn fn = fmt == QG_FMT_Q8_0 ? dense_for<QG_FMT_Q8_0>(T, rbi)
               : fmt == QG_FMT_Q4_0 ? dense_for<QG_FMT_Q4_0>(T, rbi)
                                    : dense_for<QG_FMT_BF16>(T, rbi);
    if (!fn) return (int)hipErrorInvalidValue;
    const int64_t nwg = (a.rows + tile.rows_per_wg - 1) / tile.rows_per_wg;
    hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(64 * tile.waves_per_wg), lds_bytes(tile, T), (hipStream_t)stream,
                       a);
    return (int)hipGetLastError();
}

int launch_grouped(int fmt, const Tile& tile, const GroupedArgs& a, void* stream) {
    const int rbi = rb_index(tile.rows_per_batch);
    GroupedFn fn = fmt == QG_FMT_Q8_0 ? grouped_for<QG_FMT_Q8_0>(rbi)
                 : fmt == QG_FMT_Q4_0 ? grouped_for<QG_FMT_Q4_0>(rbi)
                                      : grouped_for<QG_FMT_BF16>(rbi);
    if (!fn) return (int)hipErrorInvalidValue;
    const int64_t nwg = (int64_t)a.T * a.topk * a.tiles_per_expert;
    hipLaunchKernelGGL(fn, dim3((unsigned)nwg), dim3(64 * tile.waves_per_wg), lds_bytes(tile, a.T), (hipStream_t)stream,
                       a);
    return (int)hipGetLastError();
}

const char* hip_error_name(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace qg
