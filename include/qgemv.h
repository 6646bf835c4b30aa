/*
 * qgemv.h -- C ABI of the MI355X (gfx950) multi-token block-quantized mat-vec.
 *
 *     y[t][r] = sum_{k < cols} w[r][k] * x[t][k]        t < T (1..4), r < rows
 *
 * the product that the pages measure at 1..4 activation vectors per pass over
 * the weights: speculative-decode verify and draft steps (M5 multi-token audit,
 * "Track 2 Audit & Optimization Report: M5 Metal Kernels for Multi-Token
 * Speculative Decode", section 1 item 1 and the section 2.1 tile sweep; the M2
 * Max performance page, "Where the time goes on an M2 Max", mat-vec table).
 * Its cost is effective weight bandwidth: packed weight bytes / time per call.
 *
 * Weight formats (ggml block layouts, as the pages' format names imply):
 *   Q8_0  blocks of 32 weights: little-endian fp16 scale d, then 32 int8
 *         codes c (34 B);  w = d * c.
 *   Q4_0  blocks of 32 weights: little-endian fp16 scale d, then 16 bytes;
 *         byte j holds code j in its low nibble and code j + 16 in its high
 *         nibble (18 B, 4.5 bits per weight);  w = d * (c - 8).
 *   BF16  one little-endian bfloat16 per weight.
 * W is row-major: row r's blocks (or bf16 values) follow row r - 1's with no
 * padding; within a row the blocks run along k.
 *
 * Common conventions of the compute entry points
 *   - rows, cols: output count and reduction length (the pages write shapes as
 *     n_in x n_out; here cols = n_in, rows = n_out).
 *   - T: number of activation vectors, 1 <= T <= QG_MAX_T.
 *   - W, x, y, ids are DEVICE pointers, allocated and owned by the caller; the
 *     library allocates nothing and keeps no per-call state.
 *   - x is fp32 [T][cols] contiguous; y is fp32 [T][rows] contiguous (grouped:
 *     [T][topk][rows]).  y is overwritten (no accumulation) and must not
 *     overlap W, x or ids.
 *   - stream is a hipStream_t (NULL = the default stream).  Calls are
 *     stream-ordered and asynchronous: they return once the kernel is queued;
 *     a device fault surfaces at the caller's next synchronisation.
 *   - Every argument is checked on the host before any HIP call.  Return
 *     value: QG_OK, or a qg_status; qg_last_error() then holds a message.
 *   - Thread-safe: the only shared state is an immutable tile table and a
 *     thread-local error string.
 *   - A kernel computes each token's outputs in the same order whatever T is,
 *     so y[t] at T tokens equals y[t] at T' tokens bit for bit (the pages note
 *     that each token's sum should not depend on the token count: opus-mtp-
 *     turbo report, finding 3) when both calls run the same kind of kernel
 *     with the same k split.  The default tiles keep one kind and one k split
 *     for all T on every shape (the 248,320 x 5,120 Q8_0 LM head included);
 *     QGEMV_TILE pins a kind for every T.
 *   - Accuracy: |y - exact| <= 1e-4 * sum_k |w_k * x_k| + 1e-6 per output
 *     (fp32 accumulation of exactly decoded weights).
 *
 * Environment: QGEMV_TILE="fmt:rb,nw,rw[,k][;fmt:...]" overrides the tile for a
 * format (fmt = q8_0 | q4_0 | bf16): rb rows per lane group per batch or tile
 * (1, 2, 4, 8 or 16), nw waves per workgroup (1..12), rw rows per workgroup (a
 * multiple of 2*rb), k the kernel kind:
 *   d     each lane loads its own bytes;
 *   s     rows streamed through LDS via registers (rows of a multiple of 16 bytes);
 *   l<D>  streamed by direct-to-LDS loads, D = 2, 3, 4 or 6 tiles in flight per
 *         wave; rb 4;
 *   L<D>  as l<D>, with x staged apart;
 *   u<D>  as l<D>, waves take equal shares of (slice, tile) units; any nw;
 *   h<D>  direct-to-LDS loads on 256-wide k slices with 16 lanes per row, D = 2
 *         or 3 tiles in flight per wave; rb 4, cols a multiple of 256, nw a
 *         multiple of cols/256 (at most 12 slices); all three formats;
 *   x     matrix cores on 256-wide k slices: 16-row tiles streamed by direct-to-LDS
 *         loads, one in flight per wave, each block contracted as one bf16 matrix
 *         product against an exact three-piece split of x; rb only sets which
 *         rw are valid, cols a multiple of 256, nw a multiple of cols/256; all
 *         three formats; x2: the same with 32-row tiles (the same bits);
 *   X     x on 512-wide k slices (16 blocks a wave): cols a multiple of 512,
 *         nw a multiple of cols/512; the arithmetic of P, so the same bits as P;
 *   m     as s, contracted on the matrix cores; Q8_0 with rb 8 only;
 *   p     m in persistent form: one workgroup per CU, nw = the k slices, rw =
 *         the chunk of rows whose partial sums are buffered;
 *   P     x in persistent form on 512-wide k slices: one workgroup per CU, one
 *         16-row tile in flight per wave, nw = cols/512 (cols a multiple of
 *         512, at most 11 slices: the workgroup runs one more wave, which sums
 *         the chunks), rw = the chunk of rows (a multiple of 16) whose partial
 *         sums are buffered; rb only sets which rw are valid; all three formats.
 * A malformed or out-of-set value makes every call of that format return
 * QG_EINVAL.
 * QGEMV_P_DIRECT_STORES=1 makes kind P store each chunk's outputs as it sums them
 * instead of holding a workgroup's outputs in LDS until its end (what it does by
 * itself when they do not fit there); the bits are the same either way.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QG_OK = 0,
    QG_EINVAL = 1,       /* bad argument: null pointer, size, T, fmt, topk, bad QGEMV_TILE */
    QG_EALIGN = 2,       /* W or x not 16-byte aligned, y or ids not 4-byte aligned */
    QG_EUNSUPPORTED = 3, /* valid but not handled: BF16 cols % 8 != 0, sizes past the int32 grid */
    QG_EHIP = 4          /* the HIP runtime refused the launch */
} qg_status;

typedef enum { QG_FMT_Q8_0 = 0, QG_FMT_Q4_0 = 1, QG_FMT_BF16 = 2 } qg_format;

#define QG_MAX_T 4
#define QG_TILE_FIELDS 8 /* lanes_per_row, rows_per_batch, waves_per_wg, k_slice, rows_per_wg, mfma, kind, depth */

/* Q8_0 weights: cols % 32 == 0; W holds rows * cols/32 * 34 bytes. */
int qgemv_q8_0(int64_t rows, int64_t cols, int T, const void* W, const float* x, float* y, void* stream);

/* Q4_0 weights: cols % 32 == 0; W holds rows * cols/32 * 18 bytes. */
int qgemv_q4_0(int64_t rows, int64_t cols, int T, const void* W, const float* x, float* y, void* stream);

/* BF16 weights: cols % 8 == 0 (else QG_EUNSUPPORTED); W holds rows * cols * 2 bytes. */
int qgemv_bf16(int64_t rows, int64_t cols, int T, const void* W, const float* x, float* y, void* stream);

/*
 * Grouped experts (M5 audit, section 1 item 2: tokens grouped by expert id so
 * each distinct expert's weights are streamed once for all tokens that chose
 * it):
 *     y[t][j][r] = sum_k W_{ids[t][j]}[r][k] * x[t][k]     t < T, j < topk
 * W holds n_experts matrices of fmt, each [rows][cols], back to back; ids is
 * a DEVICE int32 [T][topk].  One launch; the grouping is done on the device.
 * An id outside [0, n_experts) cannot be reported synchronously: that slot's
 * output row y[t][j][*] is filled with NaN instead.
 */
int qgemv_grouped_experts(int fmt, int64_t n_experts, int64_t rows, int64_t cols, int T, int topk,
                          const int32_t* ids, const void* W, const float* x, float* y, void* stream);

/*
 * The expert projections of a routed-experts layer (M5 audit, section 1 item
 * 2 and the section 2.2 table: the gate/up projection and the down projection
 * of the experts the tokens picked, with tokens grouped by expert so that an
 * expert picked by several tokens is read once -- 65% overlap between the
 * tokens' expert sets in the audit's verify setting):
 *   gate/up  yg[t][j][r] = sum_k Wg_{ids[t][j]}[r][k] * x[t][k]
 *            yu[t][j][r] = sum_k Wu_{ids[t][j]}[r][k] * x[t][k]
 *            Wg and Wu are two tables like W above (rows = the experts' hidden
 *            width, cols = the model width), both streamed by one launch.
 *   down     y[t][j][r] = sum_k Wd_{ids[t][j]}[r][k] * h[t][j][k]
 *            h is a DEVICE fp32 [T][topk][cols]: one input per (token, expert)
 *            pair; the pairs naming one expert share one pass over its rows.
 * No activation is applied between them (the pages do not give it; the
 * caller computes h from yg and yu).  Conventions and errors as
 * qgemv_grouped_experts; every output must not overlap any input.
 */
int qgemv_experts_gate_up(int fmt, int64_t n_experts, int64_t rows, int64_t cols, int T, int topk, const int32_t* ids,
                          const void* Wg, const void* Wu, const float* x, float* yg, float* yu, void* stream);
int qgemv_experts_down(int fmt, int64_t n_experts, int64_t rows, int64_t cols, int T, int topk, const int32_t* ids,
                       const void* W, const float* h, float* y, void* stream);

/*
 * Fused mat-vec + argmax over rows, for the LM head that follows the verify
 * pass (the drafter-cost issue, "perf(speculative): cut the MTP drafter's
 * per-step cost...", fused LM-head / argmax proposal): for each t < T,
 *     idx[t] = the row r with the largest y[t][r] = sum_k w[r][k] * x[t][k]
 *              (ties: the lowest r),   val[t] = that y[t][r].
 * y is never written.  W, x as for the dense entry points; work (DEVICE, 8-byte
 * aligned, T uint64 values, contents overwritten), idx (DEVICE int32[T]) and
 * val (DEVICE float[T]) belong to the caller and must not overlap W, x or one
 * another.  Each y[t][r] is the same float the dense entry point computes for
 * these arguments, so idx/val equal the argmax of its output.  Needs rows of a
 * multiple of 16 bytes (else QG_EUNSUPPORTED).  Three kernel launches on
 * `stream` (clear work, mat-vec with per-workgroup maxima merged by atomic
 * max on work, unpack work into idx/val).
 */
int qgemv_argmax(int fmt, int64_t rows, int64_t cols, int T, const void* W, const float* x, void* work,
                 int32_t* idx, float* val, void* stream);

/*
 * qgemv_argmax without the work argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the per-token keys live in a library-owned device array of
 * QG_MAX_T uint64 values, one copy per GPU, set up at the first call on that GPU
 * (with it current) and held until the process ends.  The call allocates
 * nothing and calls no allocating routine.  Every call on one GPU uses that
 * GPU's array (each call clears the keys it uses first): calls that can overlap
 * in time on one GPU -- different streams, or threads without ordering -- race
 * and must not be issued.  Arguments, results, ordering and errors otherwise as
 * qgemv_argmax (T above QG_MAX_T is QG_EINVAL; QG_EHIP if the array cannot be
 * addressed on the current device).
 */
int qgemv_argmax_noalloc(int fmt, int64_t rows, int64_t cols, int T, const void* W, const float* x, int32_t* idx,
                         float* val, void* stream);

/*
 * Row subset: the mat-vec over a list of rows, for a draft-vocabulary LM head
 * that reads only the rows of the tokens the drafter may propose (the drafter-
 * cost issue, "perf(speculative): cut the MTP drafter's per-step cost...",
 * draft-vocabulary item):
 *     y[t][i] = sum_k w[ids[i]][k] * x[t][k]      t < T, i < n_sel
 * W holds all `rows` rows of fmt (as for the dense entry points); ids is a
 * DEVICE int32[n_sel] (any order, repeats allowed); y is fp32 [T][n_sel].  An id
 * outside [0, rows) cannot be reported synchronously: its output column is NaN.
 * Each y[t][i] equals the dense call's y[t][ids[i]] computed by the VALU
 * kernels.  Needs rows of a multiple of 16 bytes, cols <= 6144 (BF16: 4608)
 * and W under 2 GB (else QG_EUNSUPPORTED).
 */
int qgemv_rows(int fmt, int64_t rows, int64_t cols, int64_t n_sel, const int32_t* ids, int T, const void* W,
               const float* x, float* y, void* stream);

/*
 * Quantizers: fp32 values -> packed blocks, on the device, in the layout the
 * entry points above read.  The pages name the quantizers their weights come
 * from but not their steps (opus-mtp-turbo: Track 1 report, item 3 "Q4_0 / Q5_0
 * draft weights": Q4_0 from a "Lloyd" quantizer; "Where the time goes"
 * (meld-turbo-performance): dense projections re-encoded to Q8_0).  Per block
 * of 32 values, every decision in fp32:
 *   Q8_0             d = max|v| / 127, code = round(v * (1/d)), halves away
 *                    from zero.
 *   Q4_0 QG_Q4_ABSMAX  d = (the first element of largest magnitude, signed) / -8,
 *                    code = min(15, trunc(v * (1/d) + 8.5)); that element gets 0.
 *   Q4_0 QG_Q4_LLOYD   from the absmax codes, alternate the least-squares scale
 *                    d = sum v*(c-8) / sum (c-8)^2 (index order) and nearest-
 *                    level codes clamp(floor(v * (1/d) + 8.5), 0, 15) until the
 *                    codes repeat, at most 8 fits; d is the last fit.
 * The block stores fp16(d) (nearest, ties to even); a block whose fp16 scale
 * would be zero is stored as zeros (d = +0, codes 0 / 8).
 * src: DEVICE fp32 [rows][cols] (cols a multiple of 32); dst: DEVICE, the
 * qg_packed_bytes(fmt, rows, cols) packed bytes, overwritten.  Both 16-byte
 * aligned, not overlapping.  Non-finite inputs give unspecified bytes.
 * Stream-ordered and asynchronous like the mat-vec calls.
 */
enum { QG_Q4_ABSMAX = 0, QG_Q4_LLOYD = 1 };
int qg_quantize_q8_0(int64_t rows, int64_t cols, const float* src, void* dst, void* stream);
int qg_quantize_q4_0(int64_t rows, int64_t cols, int method, const float* src, void* dst, void* stream);

/* HBM read probe, for measurement only: reads `bytes` of src (DEVICE, 16-byte
 * aligned, bytes a positive multiple of 16) once, with coalesced 16-byte loads
 * and nothing else, using at most max_groups workgroups of 256 lanes.  It gives
 * the plain streaming-read time of a buffer, the reference the pages set their
 * mat-vec bandwidth against ("Where the time goes on an M2 Max", its bandwidth
 * table and the peak it quotes).  out: DEVICE, 4-byte aligned, not inside src;
 * written only when a wave's XOR of the words it read equals `magic` (so the
 * loads cannot be dropped), its contents otherwise unchanged.  QG_EINVAL on null
 * pointers, bad sizes or overlap; QG_EALIGN on misalignment.  Stream-ordered and
 * asynchronous. */
int qg_read_probe(const void* src, int64_t bytes, int64_t max_groups, uint32_t magic, uint32_t* out, void* stream);

/* ---- host-only helpers (no GPU needed) ---------------------------------- */

/* Packed bytes of a rows x cols matrix of fmt; 0 if the shape is invalid. */
size_t qg_packed_bytes(int fmt, int64_t rows, int64_t cols);

/* HOST pointers.  d_bits: [rows][cols/32] fp16 bit patterns; codes: [rows][cols]
 * (Q8_0 any int8, Q4_0 0..15 -- a code > 15 is QG_EINVAL).  out / in: the
 * packed bytes (qg_packed_bytes of them).  Bit-exact in both directions. */
int qg_pack_q8_0(int64_t rows, int64_t cols, const uint16_t* d_bits, const int8_t* codes, void* out);
int qg_unpack_q8_0(int64_t rows, int64_t cols, const void* in, uint16_t* d_bits, int8_t* codes);
int qg_pack_q4_0(int64_t rows, int64_t cols, const uint16_t* d_bits, const uint8_t* codes, void* out);
int qg_unpack_q4_0(int64_t rows, int64_t cols, const void* in, uint16_t* d_bits, uint8_t* codes);

/* The tile a call with these arguments would use (after QGEMV_TILE):
 * out_tile = {lanes_per_row, rows_per_batch, waves_per_wg, k_slice, rows_per_wg, mfma, kind, depth}
 * (kind 0: direct loads, 1: streamed through LDS via registers, 2 / 3: streamed
 * by direct-to-LDS loads with `depth` tiles in flight per wave (3: x staged
 * apart), 4: unit-balanced direct-to-LDS, 7: direct-to-LDS on 256-wide k slices
 * with 16 lanes per row (any format; k_slice 256, lanes_per_row 16), 8: matrix
 * cores on 256-wide k slices fed by direct-to-LDS loads (any format; k_slice 256,
 * lanes_per_row 4: a row's 32-weight block is spread over 4 lanes), 9: kind 8 in
 * persistent form on 512-wide k slices (k_slice 512, lanes_per_row 4), 11: kind 8
 * on 512-wide k slices (k_slice 512, lanes_per_row 4); mfma 1:
 * matrix-core contraction of kind 1, 2: its persistent form). */
int qg_query_tile(int fmt, int64_t rows, int64_t cols, int T, int out_tile[QG_TILE_FIELDS]);

/* Static description of a status code (never NULL). */
const char* qg_status_string(int status);

/* Detail of the calling thread's last failure ("" if none). */
const char* qg_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
