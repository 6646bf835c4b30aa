// Host front of the C ABI declared in include/qgemv.h: argument checks (all of
// them before any HIP call), the tile table and its QGEMV_TILE override, the
// bit-exact pack/unpack helpers and the status strings.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>

#include "qgemv_internal.h"

namespace qg {
namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return QG_OK;
}

bool valid_fmt(int fmt) { return fmt == QG_FMT_Q8_0 || fmt == QG_FMT_Q4_0 || fmt == QG_FMT_BF16; }

const char* fmt_name(int fmt) { return fmt == QG_FMT_Q8_0 ? "q8_0" : fmt == QG_FMT_Q4_0 ? "q4_0" : "bf16"; }

// bytes per row, -1 if cols is not whole blocks
int64_t row_bytes(int fmt, int64_t cols) {
    if (cols <= 0) return -1;
    if (fmt == QG_FMT_BF16) return cols * 2;
    if (cols % 32) return -1;
    return cols / 32 * (fmt == QG_FMT_Q8_0 ? 34 : 18);
}

// Largest sizes the kernels index with their int32 fields: cols (k positions) and
// the workgroup count; byte offsets are 64-bit throughout.
constexpr int64_t kMaxCols = int64_t(1) << 24;
constexpr int64_t kMaxRows = int64_t(1) << 31;

// "rb,nw,rw[,k]" with k = d, s, m, l<depth> or L<depth>.  Returns false (and
// the reason) when malformed or outside the compiled set.
bool parse_tile_spec(const std::string& spec, Tile* t, std::string* why) {
    int rb = 0, nw = 0, rw = 0, depth = 0;
    char kind = 0, tail = 0;
    int got = sscanf(spec.c_str(), "%d,%d,%d,%c%c", &rb, &nw, &rw, &kind, &tail);
    if (got == 5 && (kind == 'l' || kind == 'L' || kind == 'u' || kind == 'h' || kind == 'x')) {  // l|L|u|h|x<depth>
        char tail2 = 0;
        const char* f = kind == 'l' ? "%d,%d,%d,l%d%c" : kind == 'L' ? "%d,%d,%d,L%d%c"
                      : kind == 'u' ? "%d,%d,%d,u%d%c" : kind == 'h' ? "%d,%d,%d,h%d%c" : "%d,%d,%d,x%d%c";
        got = sscanf(spec.c_str(), f, &rb, &nw, &rw, &depth, &tail2) == 4 ? 4 : -1;
    }
    const bool dma = kind == 'l' || kind == 'L' || kind == 'u' || kind == 'h';
    if (!(got == 3 || (got == 4 && (kind == 'd' || kind == 's' || kind == 'm' || kind == 'p' || kind == 'P' ||
                                     kind == 'X' || (kind == 'x' && depth >= 0 && depth <= 2) || (dma && depth > 0))))) {
        *why = "tile '" + spec + "' is not rb,nw,rw[,d|s|m|p|x|x2|X|P|l<depth>|L<depth>|u<depth>|h<depth>]";
        return false;
    }
    if (!valid_rb(rb) || nw < 1 || nw > kMaxWaves || rw < 2 * rb || rw % (2 * rb) || rw > (1 << 20)) {
        *why = "tile '" + spec + "' is outside the compiled set (rb in {1,2,4,8,16}, nw in 1..12, rw a multiple of 2*rb)";
        return false;
    }
    t->rows_per_batch = rb;
    t->waves_per_wg = nw;
    t->rows_per_wg = rw;
    t->kind = got == 4 ? (kind == 'd' ? 0 : kind == 'l' ? 2 : kind == 'L' ? 3 : kind == 'u' ? 4 : kind == 'h' ? 7
                          : kind == 'x' ? 8 : kind == 'P' ? 9 : kind == 'X' ? 11 : 1)
                       : -1;  // -1: later
    t->mfma = got == 4 && kind == 'm' ? 1 : got == 4 && kind == 'p' ? 2 : 0;
    t->depth = got == 4 && dma ? depth : got == 4 && kind == 'x' ? (depth ? depth : 1)
             : got == 4 && (kind == 'P' || kind == 'X') ? 1 : 0;
    return true;
}

// ------------------------------------------------------------ tile table
// Defaults keyed by (format, rows, cols, T): measured winners for the shapes
// the pages time, then a rule for every other shape.  Every default gives each
// k slice to one wave and sums the slices in slice order, so a token's
// summation order -- and its bits -- are the same at every T.
struct TuneEntry {
    int fmt;
    int64_t rows, cols;
    int T;  // 0: every T
    const char* tile;
};
// MI355X, µs per call at T = 1..4 from sweeps over (kind, rows per workgroup,
// ring depth) where the rule's pick loses by more than a few percent.
const TuneEntry kTuned[] = {
    // 256-wide k slices on the matrix cores (one 16-row tile in flight per wave),
    // the same kind at every T; µs per call at T = 1..4 against the best earlier
    // kinds (vector-ALU, themselves one kind per shape):
    //   10240 x 2560 Q8_0: 7.6 / 7.8 / 8.0 / 8.1 (48 rows per workgroup: three
    //     full tiles per wave; 40 rows, 256 workgroups: 8.0 / 8.1 / 8.3 / 8.4)
    //     against 7.9 / 8.3 / 9.1 / 9.8 for the half-slice vector-ALU ring;
    //   2560 x 2560 Q8_0: 4.5-4.9 / 4.7-5.0 / 4.9-5.1 / 5.1-5.3 against 4.6 / 5.3 /
    //     6.2 / 6.5 (direct at T <= 3, register-streamed at T = 4);
    //   8192 x 2560 Q4_0: 6.3 / 6.5 / 6.6 / 6.9 against 6.1 / 7.2 / 8.5 / 9.5;
    //   8192 x 2560 BF16: 9.4 / 9.5 / 9.6 / 9.5 against 8.5 / 9.4 / 10.4 / 10.9 (on
    //     512-wide slices, below, 0.3 µs less again).
    {QG_FMT_Q8_0, 10240, 2560, 0, "4,10,48,x"},
    {QG_FMT_Q8_0, 2560, 2560, 0, "4,10,16,x"},
    {QG_FMT_Q4_0, 8192, 2560, 0, "4,10,32,x"},
    {QG_FMT_BF16, 8192, 2560, 0, "4,5,32,X"},  // 512-wide slices: 9.1 / 9.1 / 9.3 / 9.4 against 9.4 / 9.5 / 9.6 / 9.7
    // 2560 x 6144 Q8_0 (24 256-wide slices, more than twelve waves): the matrix cores
    // on 512-wide slices, 7.2 / 7.7 / 8.1 / 8.7 µs against 7.3 / 7.8 / 8.7 / 9.4 for the
    // register-streamed vector-ALU kernel
    {QG_FMT_Q8_0, 2560, 6144, 0, "4,12,16,X"},
    // LM head, 248,320 x 5,120 Q8_0: the persistent matrix-core kernel on the
    // LDS-DMA ring, one kind at every T, so a token's bits do not depend on T:
    // 204 / 203 / 205 / 212 µs at T = 1..4 (225 / 227 / 228 / 230 with every load
    // under the default cache policy) against 234 / 243 / 269 / 279 for the best earlier kinds
    // (the LDS-DMA vector-ALU ring at T <= 2, the persistent matrix cores with x in
    // registers at T >= 3).  Chunks of 3 or 4 tiles time alike; 2 tiles cost 1-4 µs.
    {QG_FMT_Q8_0, 248320, 5120, 0, "4,10,48,P"},
};

Tile default_tile(int fmt, int64_t rows, int64_t cols, int T) {
    Tile t{};
    t.lanes_per_row = kLanesPerRow;
    t.k_slice = kSlice;
    t.mfma = 0;
    t.depth = 0;
    const int64_t nslices = (cols + kSlice - 1) / kSlice;
    for (const TuneEntry& e : kTuned) {
        std::string why;
        if (e.fmt == fmt && e.rows == rows && e.cols == cols && (e.T == 0 || e.T == T) && parse_tile_spec(e.tile, &t, &why))
            return t;
    }
    // Q8_0 matrices about the size of the 256 MiB last-level cache or larger, up to
    // 11 512-wide slices (and a wave that sums): the persistent matrix cores on the
    // LDS-DMA ring, chunks of 3 tiles, with split loads.  µs at T = 1..4 against
    // the rule's next pick: 151,936 x 3,584 (551 MiB) 87.6 / 87.8 / 90.8 / 93.7
    // against 116 / 126 / 144 / 162 (earlier kinds); 65,536 x 5,120 (340 MiB) 60.9 /
    // 61.4 / 62.5 / 64.4 against 65.2 / 65.9 / 66.8 / 67.7; 49,152 x 5,120 (255 MiB)
    // 48.0 / 48.6 / 49.6 / 51.3 against 52.4 / 52.9 / 53.9 / 55.3; at 32,768 x 5,120
    // (170 MiB) it loses from T = 2 on (35.6 / 36.3 / 37.5 against 35.5 / 36.1 / 36.6).
    // With fewer than seven slices a CU streams too little: 100,000 x 2,560
    // (259 MiB, five slices) 49.0 / 51.2 / 53.3 / 53.6 against 46.6 / 46.9 / 47.5, so
    // below 512 MiB those stay on the next pick.
    const int64_t wbytes = rows * row_bytes(fmt, cols);
    if (fmt == QG_FMT_Q8_0 && cols % kSlice == 0 && nslices + 1 <= kMaxWaves &&
        (wbytes >= (int64_t)512 << 20 || (wbytes >= (int64_t)224 << 20 && nslices >= 7))) {
        t.kind = 9;
        t.depth = 1;
        t.rows_per_batch = 4;
        t.waves_per_wg = (int)nslices;
        t.rows_per_wg = 48;
        if (mxp_lds_bytes(fmt, t, T) <= kMaxLds) return t;
        t.kind = 0;
        t.depth = 0;
    }
    // up to 12 256-wide slices: the matrix cores, one wave per slice, about one
    // workgroup per CU in whole 16-row tiles (the tuned shapes above follow this)
    if (cols % 256 == 0 && cols / 256 <= kMaxWaves && row_bytes(fmt, cols) * 16 < 0x7FFFFFFF) {
        t.kind = 8;
        t.depth = 1;
        t.rows_per_batch = 4;
        t.waves_per_wg = (int)(cols / 256);
        int64_t rw = ((rows + 255) / 256 + 15) / 16 * 16;
        t.rows_per_wg = (int)(rw > 1024 ? 1024 : rw);
        while (t.rows_per_wg > 16 && mx_lds_bytes(fmt, t, T, t.waves_per_wg) > kMaxLds) t.rows_per_wg -= 16;
        if (mx_lds_bytes(fmt, t, T, t.waves_per_wg) <= kMaxLds) return t;
        t.kind = 0;
        t.depth = 0;
    }
    // more than 12 256-wide slices, up to 12 512-wide ones: the same on 512-wide slices
    if (cols % kSlice == 0 && nslices <= kMaxWaves && row_bytes(fmt, cols) * 16 < 0x7FFFFFFF) {
        t.kind = 11;
        t.depth = 1;
        t.rows_per_batch = 4;
        t.waves_per_wg = (int)nslices;
        int64_t rw = ((rows + 255) / 256 + 15) / 16 * 16;
        t.rows_per_wg = (int)(rw > 1024 ? 1024 : rw);
        while (t.rows_per_wg > 16 && mx_lds_bytes(fmt, t, T, (int)nslices) > kMaxLds) t.rows_per_wg -= 16;
        const bool fits = mx_lds_bytes(fmt, t, T, (int)nslices) <= kMaxLds;
        // when the LDS holds too few rows for one workgroup per CU (long matrices at
        // T >= 3, whose partial sums take more room), the persistent kind on the same
        // slices, which has the same arithmetic and so the same bits: Q4_0 248,320 x
        // 5,120 at T = 3 / 4 ran 204.5 / 206.1 µs in 388 workgroups against 176.8 /
        // 173.9 persistent (T = 1 / 2: 160.2 / 163.6 in 255 workgroups, persistent 168.2
        // / 170.5, so those stay).  BF16 (unmeasured there) keeps kind X.
        if (fits && fmt != QG_FMT_BF16 && (rows + t.rows_per_wg - 1) / t.rows_per_wg > kPersistGrid &&
            nslices + 1 <= kMaxWaves) {
            Tile p = t;
            p.kind = 9;
            p.rows_per_wg = 48;
            if (mxp_lds_bytes(fmt, p, T) <= kMaxLds) return p;
        }
        if (fits) return t;
        t.kind = 0;
        t.depth = 0;
    }
    // fewest waves that cover the slices in equal rounds
    const int64_t rounds = (nslices + kMaxWaves - 1) / kMaxWaves;
    t.waves_per_wg = (int)((nslices + rounds - 1) / rounds);
    // one batch per workgroup (every load of a wave in flight at once) when each
    // wave has one slice; otherwise the pipelined kernel with its largest batch
    const bool os = nslices <= t.waves_per_wg;
    t.kind = 0;
    const bool rows16 = row_bytes(fmt, cols) % 16 == 0;
    // rows per workgroup follow the matrix: about one workgroup per CU, in whole
    // 8-row tiles, between 16 (small matrices: fewer, fuller workgroups beat one
    // per CU) and 256 (large ones: long pipelined workgroups)
    int64_t rw = (rows / 256 + 7) / 8 * 8;
    rw = rw < 16 ? 16 : rw > 256 ? 256 : rw;
    if (os && rows16) {
        // streamed by LDS-DMA loads in 8-row tiles, one wave per k slice; the
        // ring is the smallest that leaves x its slots plus one tile (deeper
        // rings measured slower: they cost occupancy and buy nothing)
        t.kind = 2;
        t.rows_per_batch = 4;
        t.rows_per_wg = (int)rw;
        const int x_slots = dma_x_slots(fmt, T);
        for (int d : {2, 3, 4, 6}) {
            t.depth = d;
            if (d > x_slots) break;
        }
        if (dma_supported(fmt, T, 4, t.depth, false) && dma_lds_bytes(fmt, t, T, (int)nslices) <= kMaxLds) return t;
        t.depth = 0;
        t.kind = 0;
    }
    if (os && rows16 && stream_supported(fmt, T, 4)) {
        // streamed through LDS via registers, two 8-row tiles in flight
        t.kind = 1;
        t.rows_per_batch = 4;
        t.rows_per_wg = (int)(rw + 15) / 16 * 16;
        if (stream_lds_bytes(fmt, t, T, (int)nslices) <= kMaxLds) return t;
        t.rows_per_wg = 16;
        if (stream_lds_bytes(fmt, t, T, (int)nslices) <= kMaxLds) return t;
        t.kind = 0;
        t.waves_per_wg = (int)nslices;
    }
    t.rows_per_batch = 1;
    for (int rb : {2, 4, 8, os ? (T <= 2 ? 8 : 4) : 8})
        if (rb <= (os ? (T <= 2 ? 8 : 4) : 8) && tile_supported(fmt, T, rb, os)) t.rows_per_batch = rb;
    t.rows_per_wg = os ? 2 * t.rows_per_batch : 8 * t.rows_per_batch;
    return t;
}

// QGEMV_TILE="fmt:rb,nw,rw[,k][;...]".  Returns 0 (no override for fmt), 1
// (override applied to *t) or -1 (malformed / outside the compiled set).
int tile_override(int fmt, Tile* t, std::string* why) {
    const char* env = getenv("QGEMV_TILE");
    if (!env || !*env) return 0;
    std::string s(env);
    size_t pos = 0;
    while (pos <= s.size()) {
        size_t end = s.find(';', pos);
        if (end == std::string::npos) end = s.size();
        std::string item = s.substr(pos, end - pos);
        pos = end + 1;
        if (item.empty()) continue;
        size_t colon = item.find(':');
        if (colon == std::string::npos) {
            *why = "QGEMV_TILE item '" + item + "' has no 'fmt:'";
            return -1;
        }
        std::string name = item.substr(0, colon);
        int f = name == "q8_0" ? QG_FMT_Q8_0 : name == "q4_0" ? QG_FMT_Q4_0 : name == "bf16" ? QG_FMT_BF16 : -1;
        if (f < 0) {
            *why = "QGEMV_TILE format '" + name + "' unknown";
            return -1;
        }
        Tile parsed = *t;
        if (!parse_tile_spec(item.substr(colon + 1), &parsed, why)) {
            *why = "QGEMV_TILE: " + *why;
            return -1;
        }
        if (f == fmt) {
            *t = parsed;
            return 1;
        }
    }
    return 0;
}

int pick_tile(int fmt, int64_t rows, int64_t cols, int T, Tile* t) {
    *t = default_tile(fmt, rows, cols, T);
    std::string why;
    if (tile_override(fmt, t, &why) < 0) return fail(QG_EINVAL, "%s", why.c_str());
    const int64_t nslices = (cols + kSlice - 1) / kSlice;
    const bool stream_shape = row_bytes(fmt, cols) % 16 == 0 && t->waves_per_wg >= nslices &&
                              t->waves_per_wg % nslices == 0;
    if (t->kind < 0)  // override without a kind: streamed when the shape and tile allow it
        t->kind = stream_shape && stream_supported(fmt, T, t->rows_per_batch) &&
                  stream_lds_bytes(fmt, *t, T, (int)nslices) <= kMaxLds;
    if (t->kind == 4) {
        if (row_bytes(fmt, cols) % 16 != 0)
            return fail(QG_EINVAL, "streamed tile needs rows of a multiple of 16 bytes");
        if (!units_supported(t->rows_per_batch, t->depth))
            return fail(QG_EINVAL, "unit-balanced tile rb=%d depth=%d is not compiled (rb 4; depth 2..4)",
                        t->rows_per_batch, t->depth);
        if (units_lds_bytes(fmt, *t, T, cols) > kMaxLds)
            return fail(QG_EINVAL, "tile needs %zu B of LDS (x, rows_per_wg %d or depth %d too large)",
                        units_lds_bytes(fmt, *t, T, cols), t->rows_per_wg, t->depth);
        return QG_OK;
    }
    if (t->kind == 9) {
        if (cols % kSlice || t->waves_per_wg != nslices)
            return fail(QG_EINVAL, "persistent matrix-core ring tile needs cols a multiple of 512 and waves_per_wg == "
                                   "the %lld 512-wide slices", (long long)nslices);
        if (t->waves_per_wg + 1 > kMaxWaves)  // one more wave sums the chunks
            return fail(QG_EINVAL, "persistent matrix-core ring tile runs at most %d 512-wide slices (cols <= %d)",
                        kMaxWaves - 1, (kMaxWaves - 1) * (int)kSlice);
        if (t->rows_per_wg % 16)
            return fail(QG_EINVAL, "persistent matrix-core ring tile needs rows_per_wg (the chunk) a multiple of 16");
        if (row_bytes(fmt, cols) * 16 > 0x7FFFFFFF)
            return fail(QG_EINVAL, "persistent matrix-core ring tile needs 16 rows within a 2 GB descriptor");
        if (mxp_lds_bytes(fmt, *t, T) > kMaxLds)
            return fail(QG_EINVAL, "tile needs %zu B of LDS (rows_per_wg %d too large)", mxp_lds_bytes(fmt, *t, T),
                        t->rows_per_wg);
        return QG_OK;
    }
    if (t->kind == 11) {
        if (cols % kSlice || t->waves_per_wg % nslices != 0)
            return fail(QG_EINVAL, "matrix-core 512-wide-slice tile needs cols a multiple of 512 and waves_per_wg a "
                                   "multiple of the %lld 512-wide slices", (long long)nslices);
        if (row_bytes(fmt, cols) * 16 > 0x7FFFFFFF)
            return fail(QG_EINVAL, "matrix-core 512-wide-slice tile needs 16 rows within a 2 GB descriptor");
        if (mx_lds_bytes(fmt, *t, T, (int)nslices) > kMaxLds)
            return fail(QG_EINVAL, "tile needs %zu B of LDS (rows_per_wg %d too large)",
                        mx_lds_bytes(fmt, *t, T, (int)nslices), t->rows_per_wg);
        return QG_OK;
    }
    if (t->kind == 8) {
        const int64_t nsl256 = cols / 256;
        if (cols % 256 || t->waves_per_wg % nsl256 != 0)
            return fail(QG_EINVAL, "matrix-core half-slice tile needs cols a multiple of 256 and waves_per_wg a "
                                   "multiple of the %lld 256-wide slices", (long long)nsl256);
        if (row_bytes(fmt, cols) * 16 * t->depth > 0x7FFFFFFF)
            return fail(QG_EINVAL, "matrix-core half-slice tile needs %d rows within a 2 GB descriptor", 16 * t->depth);
        if (mx_lds_bytes(fmt, *t, T, (int)nsl256) > kMaxLds)
            return fail(QG_EINVAL, "tile needs %zu B of LDS (rows_per_wg %d too large)",
                        mx_lds_bytes(fmt, *t, T, (int)nsl256), t->rows_per_wg);
        return QG_OK;
    }
    if (t->kind == 7) {
        const int64_t nsl256 = cols / 256;
        if (cols % 256 || t->waves_per_wg % nsl256 != 0)
            return fail(QG_EINVAL, "half-slice tile needs cols a multiple of 256 and waves_per_wg a multiple of the "
                                   "%lld 256-wide slices", (long long)nsl256);
        if (!half_supported(t->rows_per_batch, t->depth))
            return fail(QG_EINVAL, "half-slice tile is compiled with rb 4 and depth 2 or 3");
        if (half_lds_bytes(fmt, *t, T, (int)nsl256) > kMaxLds)
            return fail(QG_EINVAL, "tile needs %zu B of LDS (rows_per_wg %d or depth %d too large)",
                        half_lds_bytes(fmt, *t, T, (int)nsl256), t->rows_per_wg, t->depth);
        return QG_OK;
    }
    if (t->kind == 2 || t->kind == 3) {
        if (!stream_shape)
            return fail(QG_EINVAL, "streamed tile needs rows of a multiple of 16 bytes and waves_per_wg a multiple of "
                                   "the %lld k slices", (long long)nslices);
        if (!dma_supported(fmt, T, t->rows_per_batch, t->depth, t->kind == 3))
            return fail(QG_EINVAL, "LDS-DMA tile rb=%d depth=%d is not compiled for this format and T=%d "
                                   "(rb 4; depth 2, 3, 4 or 6, above the %d slots x takes)",
                        t->rows_per_batch, t->depth, T, dma_x_slots(fmt, T));
        if (dma_lds_bytes(fmt, *t, T, (int)nslices) > kMaxLds)
            return fail(QG_EINVAL, "tile needs %zu B of LDS (rows_per_wg %d or depth %d too large)",
                        dma_lds_bytes(fmt, *t, T, (int)nslices), t->rows_per_wg, t->depth);
        return QG_OK;
    }
    if (t->kind == 1) {
        // waves = slices x row groups
        if (!stream_shape)
            return fail(QG_EINVAL, "streamed tile needs rows of a multiple of 16 bytes and waves_per_wg a multiple of "
                                   "the %lld k slices", (long long)nslices);
        if (t->mfma ? !mfma_supported(fmt, t->rows_per_batch) : !stream_supported(fmt, T, t->rows_per_batch))
            return fail(QG_EINVAL, "streamed%s rows_per_batch %d is not compiled for this format and T=%d",
                        t->mfma ? " matrix-core" : "", t->rows_per_batch, T);
        if (t->mfma == 2) {  // persistent: one wave per slice, rows_per_wg = buffered chunk of 16-row tiles
            if (t->waves_per_wg != nslices)
                return fail(QG_EINVAL, "persistent matrix-core tile needs waves_per_wg == the %lld k slices",
                            (long long)nslices);
            if (t->rows_per_wg % 16 != 0)
                return fail(QG_EINVAL, "persistent matrix-core tile needs rows_per_wg a multiple of 16");
            if (mfma_persist_lds_bytes(*t, T) > kMaxLds)
                return fail(QG_EINVAL, "tile needs %zu B of LDS (rows_per_wg %d too large)", mfma_persist_lds_bytes(*t, T),
                            t->rows_per_wg);
            return QG_OK;
        }
        if (stream_lds_bytes(fmt, *t, T, (int)nslices) > kMaxLds)
            return fail(QG_EINVAL, "tile needs %zu B of LDS (rows_per_wg %d too large)",
                        stream_lds_bytes(fmt, *t, T, (int)nslices), t->rows_per_wg);
        return QG_OK;
    }
    if (t->waves_per_wg > nslices) t->waves_per_wg = (int)nslices;  // idle waves would only add zeros
    if (!tile_supported(fmt, T, t->rows_per_batch, one_shot(*t, (int)nslices)))
        return fail(QG_EINVAL, "rows_per_batch %d is not compiled for T=%d with this tile", t->rows_per_batch, T);
    if (lds_bytes(*t, T) > kMaxLds)
        return fail(QG_EINVAL, "tile needs %zu B of LDS (rows_per_wg %d too large)", lds_bytes(*t, T), t->rows_per_wg);
    return QG_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

int check_common(int fmt, int64_t rows, int64_t cols, int T, const void* W, const float* x, const float* y,
                 int64_t* rb_out) {
    if (!valid_fmt(fmt)) return fail(QG_EINVAL, "unknown format %d", fmt);
    if (!W || !x || !y) return fail(QG_EINVAL, "null pointer (W=%p x=%p y=%p)", W, (const void*)x, (const void*)y);
    if (rows <= 0 || cols <= 0) return fail(QG_EINVAL, "rows=%lld cols=%lld must be positive", (long long)rows, (long long)cols);
    if (T < 1 || T > QG_MAX_T) return fail(QG_EINVAL, "T=%d outside 1..%d", T, QG_MAX_T);
    if (fmt != QG_FMT_BF16 && cols % 32) return fail(QG_EINVAL, "%s needs whole 32-weight blocks: cols=%lld", fmt_name(fmt), (long long)cols);
    if (fmt == QG_FMT_BF16 && cols % 8) return fail(QG_EUNSUPPORTED, "bf16 path needs cols %% 8 == 0: cols=%lld", (long long)cols);
    if (cols > kMaxCols || rows >= kMaxRows) return fail(QG_EUNSUPPORTED, "rows=%lld cols=%lld beyond the supported range", (long long)rows, (long long)cols);
    if (!aligned(W, 16) || !aligned(x, 16)) return fail(QG_EALIGN, "W and x must be 16-byte aligned (W=%p x=%p)", W, (const void*)x);
    if (!aligned(y, 4)) return fail(QG_EALIGN, "y must be 4-byte aligned (y=%p)", (const void*)y);
    *rb_out = row_bytes(fmt, cols);
    return QG_OK;
}

int run_dense(int fmt, int64_t rows, int64_t cols, int T, const void* W, const float* x, float* y, void* stream) {
    int64_t rbytes = 0;
    int st = check_common(fmt, rows, cols, T, W, x, y, &rbytes);
    if (st) return st;
    const size_t wbytes = (size_t)(rbytes * rows), xbytes = (size_t)T * cols * 4, ybytes = (size_t)T * rows * 4;
    if (overlap(y, ybytes, W, wbytes) || overlap(y, ybytes, x, xbytes)) return fail(QG_EINVAL, "y overlaps W or x");
    Tile tile;
    if ((st = pick_tile(fmt, rows, cols, T, &tile))) return st;
    DenseArgs a;
    a.W = (const uint8_t*)W;
    a.x = x;
    a.y = y;
    a.rows = rows;
    a.row_bytes = rbytes;
    a.cols = (int)cols;
    a.nslices = (int)((cols + kSlice - 1) / kSlice);
    a.rows_per_wg = tile.rows_per_wg;
    if ((rows + tile.rows_per_wg - 1) / tile.rows_per_wg > 0x7FFFFFFF) return fail(QG_EUNSUPPORTED, "grid too large");
    int err = tile.kind == 9   ? launch_mxp(fmt, T, tile, a, stream)
              : tile.kind == 8 || tile.kind == 11 ? launch_mx(fmt, T, tile, a, stream)
              : tile.kind == 7 ? launch_half(fmt, T, tile, a, stream)
              : tile.kind == 4 ? launch_units(fmt, T, tile, a, stream)
              : tile.kind >= 2 ? launch_dma(fmt, T, tile, a, stream)
              : tile.kind == 1 ? launch_stream(fmt, T, tile, a, stream)
                               : launch_dense(fmt, T, tile, a, stream);
    if (err) return fail(QG_EHIP, "kernel launch failed: %s", hip_error_name(err));
    return ok();
}

int run_argmax(int fmt, int64_t rows, int64_t cols, int T, const void* W, const float* x, void* work, int32_t* idx,
               float* val, void* stream) {
    int64_t rbytes = 0;
    int st = check_common(fmt, rows, cols, T, W, x, val, &rbytes);
    if (st) return st;
    if (!work || !idx) return fail(QG_EINVAL, "null pointer (work=%p idx=%p)", work, (void*)idx);
    if (!aligned(work, 8) || !aligned(idx, 4)) return fail(QG_EALIGN, "work must be 8-byte and idx 4-byte aligned");
    const size_t wbytes = (size_t)(rbytes * rows), xbytes = (size_t)T * cols * 4;
    const void* outs[3] = {work, idx, val};
    const size_t outb[3] = {(size_t)T * 8, (size_t)T * 4, (size_t)T * 4};
    for (int i = 0; i < 3; ++i) {
        if (overlap(outs[i], outb[i], W, wbytes) || overlap(outs[i], outb[i], x, xbytes))
            return fail(QG_EINVAL, "an output overlaps W or x");
        for (int j = 0; j < i; ++j)
            if (overlap(outs[i], outb[i], outs[j], outb[j])) return fail(QG_EINVAL, "work, idx and val overlap");
    }
    Tile tile;
    if ((st = pick_tile(fmt, rows, cols, T, &tile))) return st;
    const int64_t nsl = (cols + kSlice - 1) / kSlice;
    // The fused argmax runs on the persistent matrix-core, LDS-DMA (depth 2..4),
    // register-streamed (8-row tiles) and direct (rb 2) kernels, all with the
    // per-row arithmetic of the dense call; other tiles map onto one of these.
    const bool persist = tile.kind == 1 && tile.mfma == 2;
    if ((tile.kind == 2 || tile.kind == 3) && tile.depth > 4) {
        tile.depth = 4;
        if (tile.kind == 2 && !dma_supported(fmt, T, 4, 4, false)) tile.kind = 3;
        if (dma_lds_bytes(fmt, tile, T, (int)nsl) > kMaxLds) tile.kind = 0;
    }
    if (tile.kind == 7 && half_lds_bytes(fmt, tile, T, (int)(cols / 256)) > kMaxLds) tile.kind = 0;
    if (tile.kind == 8 && mx_lds_bytes(fmt, tile, T, (int)(cols / 256)) > kMaxLds) tile.kind = 0;
    if (tile.kind == 9 && mxp_lds_bytes(fmt, tile, T) > kMaxLds) tile.kind = 0;
    if (tile.kind == 11 && mx_lds_bytes(fmt, tile, T, (int)(cols / 512)) > kMaxLds) tile.kind = 0;
    if (tile.kind == 4 || (tile.kind == 1 && tile.mfma == 1)) tile.kind = 0;
    if (tile.kind == 1 && !persist && (tile.rows_per_batch != 4 || !stream_supported(fmt, T, 4))) tile.kind = 0;
    if (tile.kind == 0) {  // direct, rb 2, one wave per slice when the slices fit a workgroup
        tile.mfma = 0;
        tile.depth = 0;
        tile.rows_per_batch = 2;
        tile.waves_per_wg = (int)(nsl < kMaxWaves ? nsl : kMaxWaves);
        tile.rows_per_wg = one_shot(Tile{32, 2, tile.waves_per_wg, kSlice, 4, 0, 0, 0}, (int)nsl) ? 4 : 16;
    }
    DenseArgs a;
    a.W = (const uint8_t*)W;
    a.x = x;
    a.y = nullptr;  // never written
    a.rows = rows;
    a.row_bytes = rbytes;
    a.cols = (int)cols;
    a.nslices = (int)nsl;
    a.rows_per_wg = tile.rows_per_wg;
    if ((rows + tile.rows_per_wg - 1) / tile.rows_per_wg > 0x7FFFFFFF) return fail(QG_EUNSUPPORTED, "grid too large");
    const int err = launch_argmax(fmt, T, tile, a, work, idx, val, stream);
    if (err) return fail(QG_EHIP, "kernel launch failed: %s", hip_error_name(err));
    return ok();
}

int run_rows(int fmt, int64_t rows, int64_t cols, int64_t n_sel, const int32_t* ids, int T, const void* W,
             const float* x, float* y, void* stream) {
    int64_t rbytes = 0;
    int st = check_common(fmt, rows, cols, T, W, x, y, &rbytes);
    if (st) return st;
    if (!ids) return fail(QG_EINVAL, "null ids");
    if (n_sel < 1 || n_sel > 0x7FFFFFFF) return fail(QG_EINVAL, "n_sel=%lld must be in 1..2^31-1", (long long)n_sel);
    if (!aligned(ids, 4)) return fail(QG_EALIGN, "ids must be 4-byte aligned");
    const size_t wbytes = (size_t)(rbytes * rows), xbytes = (size_t)T * cols * 4, ybytes = (size_t)T * n_sel * 4;
    const int64_t nsl = (cols + kSlice - 1) / kSlice;
    if (rbytes % 16 != 0 || nsl > kMaxWaves)
        return fail(QG_EUNSUPPORTED, "row subset needs rows of a multiple of 16 bytes and at most %d k slices", kMaxWaves);
    if ((int64_t)wbytes >= 0x7FFFFFF0LL)
        return fail(QG_EUNSUPPORTED, "row subset addresses W with 32-bit offsets: %zu bytes is too many", wbytes);
    if (overlap(y, ybytes, W, wbytes) || overlap(y, ybytes, x, xbytes) || overlap(y, ybytes, ids, (size_t)n_sel * 4))
        return fail(QG_EINVAL, "y overlaps W, x or ids");
    // the matrix cores on 256- or 512-wide slices, as the dense call's default kinds
    // (a tile kind x or X pinned with QGEMV_TILE is taken; its rows per workgroup are
    // ids per workgroup), else the vector-ALU LDS-DMA kernel on 512-wide slices
    Tile tile{};
    tile.lanes_per_row = kLanesPerRow;
    tile.k_slice = kSlice;
    tile.rows_per_batch = 4;
    Tile pinned{};
    std::string why;
    const int ov = tile_override(fmt, &pinned, &why);
    if (ov < 0) return fail(QG_EINVAL, "%s", why.c_str());
    const int64_t nsl256 = cols / 256, nsl512 = cols / 512;
    if (ov == 1 && (pinned.kind == 8 || pinned.kind == 11)) {
        tile = pinned;
        const int64_t n = tile.kind == 11 ? nsl512 : nsl256;
        if (cols % (tile.kind == 11 ? 512 : 256) || n < 1 || tile.waves_per_wg % n || tile.depth != 1 ||
            tile.rows_per_wg % 16 || tile.rows_per_wg > 128 || mx_lds_bytes(fmt, tile, T, (int)n) > kMaxLds)
            return fail(QG_EINVAL, "row subset: pinned matrix-core tile needs 16-row tiles, at most 128 ids per "
                                   "workgroup and waves a multiple of the slices");
    } else if (ov != 1 && ((cols % 256 == 0 && nsl256 <= kMaxWaves) || (cols % 512 == 0 && nsl512 <= kMaxWaves))) {
        const bool narrow = cols % 256 == 0 && nsl256 <= kMaxWaves;
        tile.kind = narrow ? 8 : 11;
        tile.depth = 1;
        tile.waves_per_wg = (int)(narrow ? nsl256 : nsl512);
        int64_t rw = (n_sel / 256 + 15) / 16 * 16;
        tile.rows_per_wg = (int)(rw < 16 ? 16 : rw > 128 ? 128 : rw);
        while (tile.rows_per_wg > 16 && mx_lds_bytes(fmt, tile, T, tile.waves_per_wg) > kMaxLds) tile.rows_per_wg -= 16;
        if (mx_lds_bytes(fmt, tile, T, tile.waves_per_wg) > kMaxLds) tile.kind = 2;
    } else {
        tile.kind = 2;
    }
    if (tile.kind == 2) {
        tile.k_slice = kSlice;
        tile.depth = 2;
        tile.rows_per_batch = 4;
        tile.waves_per_wg = (int)nsl;
        int64_t rw = (n_sel / 256 + 7) / 8 * 8;
        tile.rows_per_wg = (int)(rw < 16 ? 16 : rw > 128 ? 128 : rw);  // two ids per lane: at most 128
        while (gather_lds_bytes(fmt, tile, T, (int)nsl) > kMaxLds && tile.rows_per_wg > 16) tile.rows_per_wg /= 2;
        if (gather_lds_bytes(fmt, tile, T, (int)nsl) > kMaxLds)
            return fail(QG_EUNSUPPORTED, "row subset: the LDS rings do not fit %lld slices of this format", (long long)nsl);
    }
    DenseArgs a;
    a.W = (const uint8_t*)W;
    a.x = x;
    a.y = y;
    a.rows = rows;
    a.row_bytes = rbytes;
    a.cols = (int)cols;
    a.nslices = (int)nsl;
    a.rows_per_wg = tile.rows_per_wg;
    const int err = launch_gather(fmt, T, tile, a, ids, n_sel, stream);
    if (err) return fail(QG_EHIP, "kernel launch failed: %s", hip_error_name(err));
    return ok();
}

// Grouped experts: one table (W), or two tables of the same shape in one launch
// (W2, outputs y2: gate and up); x per token [T][cols] or per slot
// [T][topk][cols] (per_slot: the down projection).
int run_grouped(int fmt, int64_t n_experts, int64_t rows, int64_t cols, int T, int topk, const int32_t* ids,
                const void* W, const void* W2, const float* x, float* y, float* y2, int per_slot, void* stream) {
    int64_t rbytes = 0;
    int st = check_common(fmt, rows, cols, T, W, x, y, &rbytes);
    if (st) return st;
    const int parts = W2 ? 2 : 1;
    if (W2 && (!aligned(W2, 16) || !aligned(y2, 4))) return fail(QG_EALIGN, "Wu must be 16-byte and yu 4-byte aligned");
    if (!ids) return fail(QG_EINVAL, "null ids");
    if (n_experts < 1 || n_experts > 0x7FFFFFFF) return fail(QG_EINVAL, "n_experts=%lld must be in 1..2^31-1", (long long)n_experts);
    if (topk < 1 || topk > 4096) return fail(QG_EINVAL, "topk=%d must be in 1..4096", topk);
    if (!aligned(ids, 4)) return fail(QG_EALIGN, "ids must be 4-byte aligned");
    const int64_t ebytes = rbytes * rows;
    if (ebytes > INT64_MAX / n_experts) return fail(QG_EUNSUPPORTED, "expert table too large");
    const size_t ybytes = (size_t)T * topk * rows * 4, wbytes = (size_t)(ebytes * n_experts);
    const size_t xbytes = (size_t)T * (per_slot ? topk : 1) * cols * 4;
    float* outs[2] = {y, y2};
    for (int p = 0; p < parts; ++p)
        if (overlap(outs[p], ybytes, W, wbytes) || overlap(outs[p], ybytes, x, xbytes) ||
            overlap(outs[p], ybytes, ids, (size_t)T * topk * 4) || (W2 && overlap(outs[p], ybytes, W2, wbytes)))
            return fail(QG_EINVAL, "an output overlaps W, x or ids");
    if (parts == 2 && overlap(y, ybytes, y2, ybytes)) return fail(QG_EINVAL, "yg and yu overlap");
    Tile tile;
    if ((st = pick_tile(fmt, rows, cols, QG_MAX_T, &tile))) return st;  // one kernel for 1..4 tokens per expert
    const int64_t nsl = (cols + kSlice - 1) / kSlice;
    std::string why;
    Tile probe = tile;
    const bool overridden = tile_override(fmt, &probe, &why) == 1;
    const int64_t nsl256 = cols / 256;
    const bool mx_ok = cols % 256 == 0 && nsl256 <= kMaxWaves && rbytes * 16 < 0x7FFFFFFF;
    if (!overridden && mx_ok) {
        // the matrix cores on 256-wide slices (kind 8's tiles), one wave per slice.
        // Rows per workgroup for 4 slices or more: the fewest that keep all slots' workgroups within
        // one per CU (256 experts of 512 x 2560 Q4_0, 10 slots a token, µs at
        // T = 1..4: 32 rows 7.4 / 12.9 / 13.2 / 18.8, 48 rows 8.6 / 8.8 / 15.7 / 15.9,
        // 64 rows 10.0 / 10.1 / 10.3 / 18.4, 96 rows 12.6 / 12.7 / 12.8 / 13.0: more
        // workgroups than CUs cost more than longer ones, even where two fit a CU;
        // 32-row tiles, x2, are no faster).
        tile.kind = 8;
        tile.depth = 1;
        tile.mfma = 0;
        tile.rows_per_batch = 4;
        tile.waves_per_wg = (int)nsl256;
        const int64_t slots = (int64_t)T * topk * parts;
        int64_t rw = 16;
        if (nsl256 >= 4) {
            while (rw < 512 && rw < rows && slots * ((rows + rw - 1) / rw) > kPersistGrid) rw += 16;
        } else {
            // short rows (the down projection, 2560 x 512 Q4_0): small workgroups of one
            // wave per slice, many of them per CU; 32 rows at T = 1, 64 from T = 2 (10 slots
            // a token at share 0.65, µs at T = 1..4: 6.4 / 8.2 / 9.4 / 11.2, against 6.9 /
            // 9.2 / 11.5 / 14.5 for the rule above with two row groups of waves)
            rw = (slots * rows / 800 + 15) / 16 * 16;
            rw = rw < 16 ? 16 : rw > 64 ? 64 : rw;
        }
        tile.rows_per_wg = (int)rw;
        while (tile.rows_per_wg > 16 && mx_lds_bytes(fmt, tile, T, (int)nsl256) > kMaxLds) tile.rows_per_wg -= 16;
    }
    if (tile.kind == 8) {  // default or pinned: checked as the launch needs it, else the paths below
        if (!mx_ok || tile.waves_per_wg % nsl256 || tile.rows_per_wg % 16 || rbytes * 32 * tile.depth >= 0x7FFFFFFF ||
            mx_lds_bytes(fmt, tile, T, (int)nsl256) > kMaxLds)
            tile.kind = 1;
    } else if (!overridden && row_bytes(fmt, cols) % 16 == 0 && nsl <= kMaxWaves) {
        // LDS-DMA streamed, x staged apart (any number of tokens per expert fits
        // one ring of two slots).  Rows per workgroup: the workgroups of all
        // slots (at most T * topk distinct experts) fit in about one round of
        // two workgroups per CU.
        tile.kind = 3;
        tile.depth = 2;
        tile.mfma = 0;
        tile.rows_per_batch = 4;
        // fewer than 4 k slices (the down projection's short rows): row groups of
        // waves share the workgroup's rows, 4 waves or more in all
        const int64_t rg = nsl >= 4 ? 1 : (4 + nsl - 1) / nsl;
        tile.waves_per_wg = (int)(nsl * rg);
        // (at least 24 rows, 3 tiles, for full-length rows: one token's 10 experts of
        // 512 rows ran 8.9 us in 220 workgroups of 24 rows against 9.4 in 320 of 16)
        int64_t rw = ((int64_t)T * topk * parts * rows / 480 + 7) / 8 * 8;
        const int64_t rw_min = rg == 1 ? 24 : 16 * rg;
        tile.rows_per_wg = (int)(rw < rw_min ? rw_min : rw > 256 ? 256 : rw);
        if (dma_lds_bytes(fmt, tile, T, (int)nsl) > kMaxLds) tile.kind = 1;  // fall back below
    }
    if (tile.kind == 2 || tile.kind == 3) {  // any DMA tile runs the grouped DMA kernel, x staged apart
        tile.kind = 3;
        if (tile.depth != 3) tile.depth = 2;
        if (tile.waves_per_wg % nsl != 0 || dma_lds_bytes(fmt, tile, T, (int)nsl) > kMaxLds) tile.kind = 1;
    }
    if (tile.kind != 0 && tile.kind != 3 && tile.kind != 8) {  // the grouped kernel runs the direct path: one wave per slice
        tile.kind = 0;
        tile.depth = 0;
        tile.mfma = 0;
        if (tile.waves_per_wg > nsl) tile.waves_per_wg = (int)nsl;
        tile.rows_per_wg = 2 * tile.rows_per_batch;
        if (!tile_supported(fmt, QG_MAX_T, tile.rows_per_batch, one_shot(tile, (int)((cols + kSlice - 1) / kSlice))))
            tile.rows_per_batch = 2, tile.rows_per_wg = 4;
    }
    GroupedArgs a;
    a.W = (const uint8_t*)W;
    a.x = x;
    a.y = y;
    a.ids = ids;
    a.rows = rows;
    a.row_bytes = rbytes;
    a.expert_bytes = ebytes;
    a.n_experts = (int)n_experts;
    a.cols = (int)cols;
    a.nslices = (int)((cols + kSlice - 1) / kSlice);
    a.rows_per_wg = tile.rows_per_wg;
    a.tiles_per_expert = (int)((rows + tile.rows_per_wg - 1) / tile.rows_per_wg);
    a.T = T;
    a.topk = topk;
    a.W2 = (const uint8_t*)W2;
    a.y2 = y2;
    a.parts = parts;
    a.per_slot_x = per_slot;
    if ((int64_t)T * topk * a.tiles_per_expert * parts > 0x7FFFFFFF) return fail(QG_EUNSUPPORTED, "grid too large");
    int err = launch_grouped(fmt, tile, a, stream);
    if (err) return fail(QG_EHIP, "kernel launch failed: %s", hip_error_name(err));
    return ok();
}

// Quantizers: kind 0 Q8_0, 1 Q4_0 absmax, 2 Q4_0 Lloyd.
int run_quantize(int kind, int64_t rows, int64_t cols, const float* src, void* dst, void* stream) {
    const char* name = kind == 0 ? "qg_quantize_q8_0" : "qg_quantize_q4_0";
    if (!src || !dst) return fail(QG_EINVAL, "%s: null pointer (src=%p dst=%p)", name, (const void*)src, dst);
    if (rows <= 0 || cols <= 0) return fail(QG_EINVAL, "rows=%lld cols=%lld must be positive", (long long)rows, (long long)cols);
    if (cols % 32) return fail(QG_EINVAL, "%s needs whole 32-value blocks: cols=%lld", name, (long long)cols);
    if (cols > kMaxCols || rows >= kMaxRows)
        return fail(QG_EUNSUPPORTED, "rows=%lld cols=%lld beyond the supported range", (long long)rows, (long long)cols);
    if (!aligned(src, 16) || !aligned(dst, 16))
        return fail(QG_EALIGN, "src and dst must be 16-byte aligned (src=%p dst=%p)", (const void*)src, dst);
    const int64_t nblocks = rows * (cols / 32);
    if ((nblocks + 255) / 256 > 0x7FFFFFFF) return fail(QG_EUNSUPPORTED, "grid too large");
    if (overlap(src, (size_t)nblocks * 128, dst, (size_t)nblocks * (kind == 0 ? 34 : 18)))
        return fail(QG_EINVAL, "dst overlaps src");
    const int err = launch_quantize(kind, src, (uint8_t*)dst, nblocks, stream);
    if (err) return fail(QG_EHIP, "kernel launch failed: %s", hip_error_name(err));
    return ok();
}

int run_read_probe(const void* src, int64_t bytes, int64_t max_groups, uint32_t magic, uint32_t* out, void* stream) {
    if (!src || !out) return fail(QG_EINVAL, "qg_read_probe: null pointer (src=%p out=%p)", src, (void*)out);
    if (bytes <= 0 || bytes % 16) return fail(QG_EINVAL, "qg_read_probe: bytes=%lld must be a positive multiple of 16", (long long)bytes);
    if (max_groups < 1 || max_groups > 0x7FFFFFFF)
        return fail(QG_EINVAL, "qg_read_probe: max_groups=%lld outside 1..2^31-1", (long long)max_groups);
    if (!aligned(src, 16) || !aligned(out, 4)) return fail(QG_EALIGN, "qg_read_probe: src must be 16-byte, out 4-byte aligned");
    if (overlap(out, 4, src, (size_t)bytes)) return fail(QG_EINVAL, "qg_read_probe: out overlaps src");
    const int err = launch_read_probe(src, bytes, max_groups, magic, out, stream);
    if (err) return fail(QG_EHIP, "kernel launch failed: %s", hip_error_name(err));
    return ok();
}

}  // namespace
}  // namespace qg

using namespace qg;

extern "C" {

int qgemv_q8_0(int64_t rows, int64_t cols, int T, const void* W, const float* x, float* y, void* stream) {
    return run_dense(QG_FMT_Q8_0, rows, cols, T, W, x, y, stream);
}

int qgemv_q4_0(int64_t rows, int64_t cols, int T, const void* W, const float* x, float* y, void* stream) {
    return run_dense(QG_FMT_Q4_0, rows, cols, T, W, x, y, stream);
}

int qgemv_bf16(int64_t rows, int64_t cols, int T, const void* W, const float* x, float* y, void* stream) {
    return run_dense(QG_FMT_BF16, rows, cols, T, W, x, y, stream);
}

int qgemv_rows(int fmt, int64_t rows, int64_t cols, int64_t n_sel, const int32_t* ids, int T, const void* W,
               const float* x, float* y, void* stream) {
    return run_rows(fmt, rows, cols, n_sel, ids, T, W, x, y, stream);
}

int qgemv_argmax(int fmt, int64_t rows, int64_t cols, int T, const void* W, const float* x, void* work, int32_t* idx,
                 float* val, void* stream) {
    return run_argmax(fmt, rows, cols, T, W, x, work, idx, val, stream);
}

int qgemv_argmax_noalloc(int fmt, int64_t rows, int64_t cols, int T, const void* W, const float* x, int32_t* idx,
                         float* val, void* stream) {
    // every argument is checked before the first HIP call (the scratch lookup)
    int64_t rbytes = 0;
    int st = check_common(fmt, rows, cols, T, W, x, val, &rbytes);
    if (st) return st;
    if (!idx) return fail(QG_EINVAL, "null idx");
    if (!aligned(idx, 4)) return fail(QG_EALIGN, "idx must be 4-byte aligned");
    void* keys = nullptr;
    const int err = argmax_scratch(&keys);
    if (err) return fail(QG_EHIP, "device scratch of the argmax keys not addressable: %s", hip_error_name(err));
    return run_argmax(fmt, rows, cols, T, W, x, keys, idx, val, stream);
}

int qgemv_grouped_experts(int fmt, int64_t n_experts, int64_t rows, int64_t cols, int T, int topk,
                          const int32_t* ids, const void* W, const float* x, float* y, void* stream) {
    return run_grouped(fmt, n_experts, rows, cols, T, topk, ids, W, nullptr, x, y, nullptr, 0, stream);
}

int qgemv_experts_gate_up(int fmt, int64_t n_experts, int64_t rows, int64_t cols, int T, int topk, const int32_t* ids,
                          const void* Wg, const void* Wu, const float* x, float* yg, float* yu, void* stream) {
    if (!Wu || !yu) return fail(QG_EINVAL, "null pointer (Wu=%p yu=%p)", Wu, (void*)yu);
    return run_grouped(fmt, n_experts, rows, cols, T, topk, ids, Wg, Wu, x, yg, yu, 0, stream);
}

int qgemv_experts_down(int fmt, int64_t n_experts, int64_t rows, int64_t cols, int T, int topk, const int32_t* ids,
                       const void* W, const float* h, float* y, void* stream) {
    return run_grouped(fmt, n_experts, rows, cols, T, topk, ids, W, nullptr, h, y, nullptr, 1, stream);
}

int qg_read_probe(const void* src, int64_t bytes, int64_t max_groups, uint32_t magic, uint32_t* out, void* stream) {
    return run_read_probe(src, bytes, max_groups, magic, out, stream);
}

int qg_quantize_q8_0(int64_t rows, int64_t cols, const float* src, void* dst, void* stream) {
    return run_quantize(0, rows, cols, src, dst, stream);
}

int qg_quantize_q4_0(int64_t rows, int64_t cols, int method, const float* src, void* dst, void* stream) {
    if (method != QG_Q4_ABSMAX && method != QG_Q4_LLOYD) return fail(QG_EINVAL, "unknown Q4_0 method %d", method);
    return run_quantize(method == QG_Q4_ABSMAX ? 1 : 2, rows, cols, src, dst, stream);
}

size_t qg_packed_bytes(int fmt, int64_t rows, int64_t cols) {
    if (!valid_fmt(fmt) || rows < 0) return 0;
    const int64_t rb = row_bytes(fmt, cols);
    if (rb < 0 || (rows && rb > INT64_MAX / rows)) return 0;
    return (size_t)(rb * rows);
}

int qg_pack_q8_0(int64_t rows, int64_t cols, const uint16_t* d_bits, const int8_t* codes, void* out) {
    if (rows < 0 || cols <= 0 || cols % 32 || !d_bits || !codes || !out) return fail(QG_EINVAL, "bad arguments to qg_pack_q8_0");
    const int64_t nb = cols / 32;
    uint8_t* o = (uint8_t*)out;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            uint8_t* blk = o + (r * nb + b) * 34;
            const uint16_t d = d_bits[r * nb + b];
            blk[0] = (uint8_t)(d & 0xFF);
            blk[1] = (uint8_t)(d >> 8);
            memcpy(blk + 2, codes + r * cols + b * 32, 32);
        }
    return ok();
}

int qg_unpack_q8_0(int64_t rows, int64_t cols, const void* in, uint16_t* d_bits, int8_t* codes) {
    if (rows < 0 || cols <= 0 || cols % 32 || !in || !d_bits || !codes) return fail(QG_EINVAL, "bad arguments to qg_unpack_q8_0");
    const int64_t nb = cols / 32;
    const uint8_t* p = (const uint8_t*)in;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t* blk = p + (r * nb + b) * 34;
            d_bits[r * nb + b] = (uint16_t)(blk[0] | (blk[1] << 8));
            memcpy(codes + r * cols + b * 32, blk + 2, 32);
        }
    return ok();
}

int qg_pack_q4_0(int64_t rows, int64_t cols, const uint16_t* d_bits, const uint8_t* codes, void* out) {
    if (rows < 0 || cols <= 0 || cols % 32 || !d_bits || !codes || !out) return fail(QG_EINVAL, "bad arguments to qg_pack_q4_0");
    for (int64_t i = 0; i < rows * cols; ++i)
        if (codes[i] > 15) return fail(QG_EINVAL, "q4_0 code %u at %lld is not 0..15", codes[i], (long long)i);
    const int64_t nb = cols / 32;
    uint8_t* o = (uint8_t*)out;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            uint8_t* blk = o + (r * nb + b) * 18;
            const uint16_t d = d_bits[r * nb + b];
            const uint8_t* c = codes + r * cols + b * 32;
            blk[0] = (uint8_t)(d & 0xFF);
            blk[1] = (uint8_t)(d >> 8);
            for (int j = 0; j < 16; ++j) blk[2 + j] = (uint8_t)(c[j] | (c[j + 16] << 4));
        }
    return ok();
}

int qg_unpack_q4_0(int64_t rows, int64_t cols, const void* in, uint16_t* d_bits, uint8_t* codes) {
    if (rows < 0 || cols <= 0 || cols % 32 || !in || !d_bits || !codes) return fail(QG_EINVAL, "bad arguments to qg_unpack_q4_0");
    const int64_t nb = cols / 32;
    const uint8_t* p = (const uint8_t*)in;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t* blk = p + (r * nb + b) * 18;
            uint8_t* c = codes + r * cols + b * 32;
            d_bits[r * nb + b] = (uint16_t)(blk[0] | (blk[1] << 8));
            for (int j = 0; j < 16; ++j) {
                c[j] = blk[2 + j] & 15;
                c[j + 16] = blk[2 + j] >> 4;
            }
        }
    return ok();
}

int qg_query_tile(int fmt, int64_t rows, int64_t cols, int T, int out_tile[QG_TILE_FIELDS]) {
    if (!valid_fmt(fmt) || rows <= 0 || cols <= 0 || T < 1 || T > QG_MAX_T || !out_tile)
        return fail(QG_EINVAL, "bad arguments to qg_query_tile");
    Tile t;
    int st = pick_tile(fmt, rows, cols, T, &t);
    if (st) return st;
    const bool half = t.kind == 7 || t.kind == 8;  // 256-wide k slices
    out_tile[0] = t.kind >= 8 ? 4 : half ? 16 : t.lanes_per_row;  // kinds 8, 9, 11: a row's block sits in 4 lanes
    out_tile[1] = t.rows_per_batch;
    out_tile[2] = t.waves_per_wg;
    out_tile[3] = half ? 256 : t.k_slice;
    out_tile[4] = t.rows_per_wg;
    out_tile[5] = t.mfma;
    out_tile[6] = t.kind;
    out_tile[7] = t.depth;
    return ok();
}

const char* qg_status_string(int status) {
    switch (status) {
    case QG_OK: return "QG_OK: success";
    case QG_EINVAL: return "QG_EINVAL: invalid argument";
    case QG_EALIGN: return "QG_EALIGN: misaligned pointer";
    case QG_EUNSUPPORTED: return "QG_EUNSUPPORTED: valid but unsupported shape";
    case QG_EHIP: return "QG_EHIP: HIP runtime error";
    }
    return "unknown qgemv status";
}

const char* qg_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
