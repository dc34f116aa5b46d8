// Host side of libfd: argument checking, the split-count planner, workspace
// layout and kernel dispatch.  No device memory is allocated here and no call
// synchronises; kernels are launched on the caller's stream.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <mutex>

#include "fd_kernels.h"

namespace {

thread_local char g_err[512] = "";

fd_status_t fail(fd_status_t st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

fd_status_t hip_fail(hipError_t e, const char *what) {
    return fail(FD_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

inline bool is_pow2(long x) { return x > 0 && (x & (x - 1)) == 0; }
inline long ceil_div(long a, long b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline int ilog2(int x) { int r = 0; while ((1 << r) < x) ++r; return r; }

// Integer environment override (experiments only); malformed values and
// negatives fall back to the default.
long env_long(const char *name, long dflt) {
    const char *s = std::getenv(name);
    if (!s || !*s) return dflt;
    char *end = nullptr;
    const long v = std::strtol(s, &end, 10);
    return (end && *end == '\0' && v >= 0) ? v : dflt;
}

constexpr uint32_t kOptionsV1 = sizeof(fd_options_t);
constexpr int kMaxQueries = 65536;       // queries per sequence
constexpr int kMaxDecodeQueries = 16;    // more take the query-tiled (prefill) kernel
// More query rows per kv head than this take the query-tiled kernel too
// (f16 / bf16), which reads K/V once for a tile of 64 or 128 rows.  The
// matrix-core split kernel holds 32 rows in one K/V read (two 16-row
// blocks, value product on 16x16x32 MFMAs), and there it is the faster one
// (measured, bf16, 8 causal queries x 4 heads: GQA 128k 330 vs 368-376 us,
// paged ragged batch 402 vs 480 us; 5 queries x 4 heads: 321 vs 367 us and
// 388 vs 488 us; B=64 with 4 queries: 1225 vs 1432 us).
constexpr int kMaxSplitRows = 32;
// bf16 V is converted to f16 for the query-tiled kernel's value product
// from this many query rows per kv head: the conversion reads V twice and
// writes it once, which the cheaper product repays only when many rows
// share each V tile (measured crossover near 1024 rows).
constexpr int kConvertRows = 1024;
// K/V bytes of a call (its longest sequence for every one) up to which the
// automatic plan merges splits in the launch (see make_plan).
constexpr double kFusedMaxBytes = 48.0 * (1 << 20);

// Compute units of the current device, cached per device id.
fd_status_t device_cus(int *cus) {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev >= 0 && dev < 64) {
        std::lock_guard<std::mutex> lock(mu);
        if (cache[dev] > 0) { *cus = cache[dev]; return FD_OK; }
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(MultiprocessorCount)");
    if (n <= 0) return fail(FD_ERR_HIP, "device reports %d compute units", n);
    if (dev >= 0 && dev < 64) {
        std::lock_guard<std::mutex> lock(mu);
        cache[dev] = n;
    }
    *cus = n;
    return FD_OK;
}

fd_status_t read_options(const fd_options_t *opt, fd_options_t *o) {
    if (!opt) return fail(FD_ERR_INVALID_ARG, "options pointer is NULL (use fd_options_init)");
    if (opt->struct_size < kOptionsV1)
        return fail(FD_ERR_INVALID_ARG, "options struct_size %u < %u", opt->struct_size, kOptionsV1);
    std::memcpy(o, opt, kOptionsV1);
    if (o->dtype != FD_F32 && o->dtype != FD_F16 && o->dtype != FD_BF16)
        return fail(FD_ERR_INVALID_ARG, "unknown dtype %d", (int)o->dtype);
    if (o->path != FD_PATH_AUTO && o->path != FD_PATH_VALU && o->path != FD_PATH_MFMA && o->path != FD_PATH_PREFILL)
        return fail(FD_ERR_INVALID_ARG, "unknown path %d", (int)o->path);
    if (o->num_cus < 0) return fail(FD_ERR_INVALID_ARG, "num_cus %d < 0", (int)o->num_cus);
    if (o->flags & ~(FD_FLAG_FUSED_MERGE | FD_FLAG_COMBINE_KERNEL | FD_FLAG_APPEND))
        return fail(FD_ERR_INVALID_ARG, "unknown flags 0x%x", (unsigned)o->flags);
    if ((o->flags & FD_FLAG_FUSED_MERGE) && (o->flags & FD_FLAG_COMBINE_KERNEL))
        return fail(FD_ERR_INVALID_ARG, "FD_FLAG_FUSED_MERGE and FD_FLAG_COMBINE_KERNEL exclude each other");
    if (o->n_queries == 0) o->n_queries = 1;
    if (o->n_queries < 1 || o->n_queries > kMaxQueries)
        return fail(FD_ERR_INVALID_ARG, "n_queries=%d not in [1, %d]", (int)o->n_queries, kMaxQueries);
    if (o->causal != 0 && o->causal != 1) return fail(FD_ERR_INVALID_ARG, "causal=%d is not 0 or 1", (int)o->causal);
    if ((o->flags & FD_FLAG_APPEND) && o->n_queries > 1)
        return fail(FD_ERR_UNSUPPORTED, "fd_append_decode takes one query per sequence");
    return FD_OK;
}

// Ragged (paged) query-tiled calls with one row tile per kv head and
// several splits run their (sequence, split) columns longest first: the
// full-length splits, then each sequence's last, partial one by size, so
// the dispatch ends on short work (measured on the paged ragged batch with
// 16 causal queries; FD_PREFILL_ORDER=0 keeps the plain order).
bool prefill_ordered(bool paged, long tiles, long n_splits, int B) {
    return paged && tiles == 1 && n_splits > 1 && n_splits < 65536 && B <= fdk::kOrderMaxB &&
           env_long("FD_PREFILL_ORDER", 1) == 1;
}

// Ordered calls with the automatic split count also let the order pass pick
// the chunk from the lengths (the host plans for T only): the plan then has
// twice the columns a length-blind plan would use, and its chunk is the
// smallest the pass may pick (FD_PREFILL_DEVCHUNK=0: the plan's chunk).
bool prefill_devchunk(bool ordered, int n_req) {
    return ordered && n_req == 0 && env_long("FD_PREFILL_DEVCHUNK", 1) == 1;
}

// Shape checks and the plan.  `paged` tells whether a page table is used.
fd_status_t make_plan(int B, int Hq, int Hkv, int T, int D, int n_req, const fd_options_t &o,
                      bool paged, fd_plan_t *p) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || T <= 0)
        return fail(FD_ERR_INVALID_ARG, "B=%d Hq=%d Hkv=%d T=%d must all be positive", B, Hq, Hkv, T);
    if (Hq % Hkv != 0) return fail(FD_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (D <= 0) return fail(FD_ERR_INVALID_ARG, "D=%d must be positive", D);
    if (D != 64 && D != 128) return fail(FD_ERR_UNSUPPORTED, "D=%d (supported: 64, 128)", D);
    if (n_req < 0) return fail(FD_ERR_INVALID_ARG, "n_splits=%d < 0", n_req);
    if (B > 65535) return fail(FD_ERR_UNSUPPORTED, "B=%d > 65535", B);
    if ((long)B * Hq * o.n_queries > (1L << 30)) return fail(FD_ERR_UNSUPPORTED, "B*n_queries*Hq too large");
    if (paged) {
        if (!is_pow2(o.page_size) || o.page_size > 65536)
            return fail(FD_ERR_INVALID_ARG, "page_size=%d is not a power of two in [1, 65536]", o.page_size);
        if (o.max_pages_per_seq < ceil_div(T, o.page_size))
            return fail(FD_ERR_INVALID_ARG, "max_pages_per_seq=%d < ceil(T/page_size)=%ld",
                        o.max_pages_per_seq, ceil_div(T, o.page_size));
        if (o.num_pages <= 0) return fail(FD_ERR_INVALID_ARG, "num_pages=%d must be positive", o.num_pages);
    }
    const long elt = o.dtype == FD_F32 ? 4 : 2;
    if (!paged && (long)T * D * elt >= (1L << 32))
        return fail(FD_ERR_UNSUPPORTED, "one (batch, kv head) cache slice of T*D*%ld bytes must be < 4 GiB", elt);

    // Path: the matrix-core kernel once a kv head's query group makes the
    // logit and value updates real small-M contractions (f16 / bf16 only).
    const int G = Hq / Hkv;
    const int R = o.n_queries * G;       // query rows per kv head
    int path = o.path;

    // Many queries per sequence (prefill), or more query rows per kv head
    // than one matrix-core split workgroup holds: the query-tiled kernel,
    // one workgroup per tile of query rows and split of the KV axis.  The
    // KV axis is split only when the row tiles alone give the device too
    // few workgroups (few queries over a long cache; a ragged batch, whose
    // lengths the host does not see, is planned for its longest sequence).
    // bf16 inputs with many rows take a workspace for V converted to f16
    // (two passes ahead of the kernel); with fewer, V is read as given and
    // P enters the value product in two bf16 parts.  FD_PREFILL_VT=0 / 1
    // forces either form.
    const bool many_rows = o.dtype != FD_F32 && R > kMaxSplitRows && !(o.flags & FD_FLAG_APPEND);
    if (path == FD_PATH_PREFILL ||
        (path == FD_PATH_AUTO && (o.n_queries > kMaxDecodeQueries || many_rows))) {
        if (o.dtype == FD_F32) return fail(FD_ERR_UNSUPPORTED, "the query-tiled kernel needs f16 or bf16 inputs");
        if (o.flags & FD_FLAG_APPEND) return fail(FD_ERR_UNSUPPORTED, "fd_append_decode takes one query per sequence");
        if (Hkv > 65535) return fail(FD_ERR_UNSUPPORTED, "Hkv=%d > 65535", Hkv);
        const bool vt = o.dtype == FD_BF16 && env_long("FD_PREFILL_VT", R >= kConvertRows ? 1 : 0) == 1;
        // 64-row tiles for up to 64 rows (no idle row blocks), else 128
        const int tile_rows = (R <= fdk::kPrefillSmallRows && !vt && env_long("FD_PREFILL_SMALL", 1) == 1)
                                  ? fdk::kPrefillSmallRows
                                  : fdk::kPrefillRows;
        const long tiles = ceil_div(R, tile_rows);
        // the converted V of one (batch, kv head) is addressed with 32-bit
        // offsets, as contiguous slices are
        if (vt && ceil_div(T, fdk::kPrefillTokens) * fdk::kPrefillTokens * D * 2 >= (1L << 32))
            return fail(FD_ERR_UNSUPPORTED, "T=%d: the converted V of one (batch, kv head) must be < 4 GiB", T);
        const long ntiles = ceil_div(T, fdk::kPrefillTokens);   // KV tiles of the longest sequence
        long n = 1;
        if (n_req > 0) {
            n = n_req < ntiles ? n_req : ntiles;
        } else {
            int cus = o.num_cus;
            if (cus == 0) {
                fd_status_t st = device_cus(&cus);
                if (st != FD_OK) return st;
            }
            // Several row tiles per kv head (bound by the matrix cores), or
            // a paged (ragged) batch: enough workgroups for about four
            // rounds at two per compute unit, so that ragged lengths and
            // causal triangles even out -- unless the row tiles alone give
            // two such rounds (measured: splitting 1024 workgroups of MHA
            // 4096-query prefill in two added 40% for the merge).  One row
            // tile of a contiguous cache
            // (a few queries: bound by K/V reads): about two rounds, as
            // longer splits stream more efficiently, and no split at all
            // once the row tiles give two workgroups per compute unit (the
            // kernel's occupancy; measured 2-3% faster than two splits and
            // the merge).  No split shorter than min_chunk tokens (its
            // pipeline fill and partial write stay small against its work).
            const long units = (long)B * Hkv * tiles;
            const bool streaming = tiles == 1 && !paged;
            long dflt = (streaming ? 4L : 8L) * cus;
            if (units >= (streaming ? 2L : 4L) * cus) dflt = units;
            const long target = std::max(1L, env_long("FD_PREFILL_WGS", dflt));
            const long min_chunk = std::max((long)fdk::kPrefillTokens, env_long("FD_PREFILL_CHUNK_MIN", 1024));
            if (units < target) {
                n = ceil_div(target, units);
                const long cap = std::max(1L, (long)T / min_chunk);
                if (n > cap) n = cap;
            }
        }
        long chunk = ceil_div(ceil_div(T, n), fdk::kPrefillTokens) * fdk::kPrefillTokens;
        n = ceil_div(T, chunk);
        if (prefill_devchunk(prefill_ordered(paged, tiles, n, B), n_req)) {
            const long ntiles_t = ceil_div(T, fdk::kPrefillTokens);
            const long ncap = std::min(2 * n, ntiles_t);
            chunk = ceil_div(ntiles_t, ncap) * fdk::kPrefillTokens;
            n = ceil_div(T, chunk);
        }
        if (tiles * n * Hkv * B > 0x7fffffffL) return fail(FD_ERR_UNSUPPORTED, "too many query-tiled workgroups");
        std::memset(p, 0, sizeof *p);
        p->n_splits = (int)n;
        p->chunk = (int)(n > 1 ? chunk : T);
        p->path = FD_PATH_PREFILL;
        p->tile = fdk::kPrefillTokens;
        p->heads_per_block = tile_rows;
        p->head_blocks = (int)tiles;
        p->grid[0] = (int)(tiles * n);
        p->grid[1] = Hkv;
        p->grid[2] = B;
        p->block = 256;
        p->combine = n > 1;
        if (vt) p->workspace_bytes = fdk::prefill_vt_bytes(B, Hkv, T, D);
        p->workspace_bytes += fdk::prefill_part_bytes(B, Hkv, R, D, (int)n);
        if (prefill_ordered(paged, tiles, n, B)) p->workspace_bytes += fdk::prefill_order_bytes(B, (int)n);
        return FD_OK;
    }
    if (o.n_queries > kMaxDecodeQueries)
        return fail(FD_ERR_UNSUPPORTED, "more than %d queries per sequence take the query-tiled path", kMaxDecodeQueries);
    if (path == FD_PATH_MFMA && o.dtype == FD_F32)
        return fail(FD_ERR_UNSUPPORTED, "the MFMA path needs f16 or bf16 inputs");
    if (path == FD_PATH_AUTO) {
        // Measured: the matrix-core kernel wins from G = 4.  With an
        // explicit split count on a paged (ragged) batch, whose short splits
        // expose the per-workgroup pipeline fill, the VALU kernel's higher
        // occupancy wins at G = 4; the automatic paged plan uses the
        // balanced stream mode instead.
        const long min_g = env_long("FD_MFMA_MIN_G", (paged && n_req > 0) ? 8 : 4);
        path = (o.dtype != FD_F32 && R >= min_g) ? FD_PATH_MFMA : FD_PATH_VALU;
    }
    int hpb, tile;
    if (path == FD_PATH_MFMA) {
        // 16 query rows per workgroup, or 32 (two row blocks on one K / V
        // read) when a kv head has more than 16
        hpb = R > fdk::kMfmaHeads ? 2 * fdk::kMfmaHeads : fdk::kMfmaHeads;
        tile = fdk::kMfmaTile;
    } else {
        hpb = 1;
        while (hpb < R && hpb < 8) hpb <<= 1;
        tile = fdk::valu_tile(o.dtype, D, hpb);
    }
    const int head_blocks = (int)ceil_div(R, hpb);
    if ((long)Hkv * head_blocks > 65535) return fail(FD_ERR_UNSUPPORTED, "Hkv*head_blocks > 65535");
    if (tile <= 0) return fail(FD_ERR_UNSUPPORTED, "no kernel instance for this shape");

    int cus = o.num_cus;
    if (cus == 0) {
        fd_status_t st = device_cus(&cus);
        if (st != FD_OK) return st;
    }

    std::memset(p, 0, sizeof *p);

    // Stream mode for ragged (paged) batches: the rows are laid end to end
    // and cut into one equal range per resident workgroup, so sequences of
    // any lengths spread evenly and no workgroup is launched for an empty
    // split.  Taken on the automatic split count only; an explicit n_splits
    // keeps the split grid.
    // One workgroup per compute unit: with two, the one dispatched second
    // to a compute unit was measured to stream its equal share ~26% slower
    // (the older waves win issue), and the call waits for it (paged ragged
    // batch: 370.5 us with one per compute unit, 387.3 us with two; an
    // 8-wave workgroup per compute unit, 388 us).
    const bool stream = paged && n_req == 0 && B <= fdk::kStreamMaxB && env_long("FD_STREAM", 1) == 1;
    if (stream) {
        const long rows = (long)B * Hkv * head_blocks;
        const long nw = std::max(1L, env_long("FD_STREAM_WGS", (long)cus));
        p->n_splits = (int)nw;
        p->chunk = 0;
        p->path = path;
        p->tile = tile;
        p->heads_per_block = hpb;
        p->head_blocks = head_blocks;
        p->grid[0] = (int)nw;
        p->grid[1] = 1;
        p->grid[2] = 1;
        p->block = 256;
        p->combine = 1;
        p->fused = 1;
        p->stream = 1;
        const size_t slots = (size_t)(rows + nw) * hpb;
        p->workspace_bytes = align256(rows * 2 * sizeof(unsigned long long)) + align256(slots * D * sizeof(float)) +
                             2 * align256(slots * sizeof(float));
        if (FD_WG_TIMING) p->workspace_bytes += align256((size_t)nw * fdk::kWgClockSlots * 8);
        return FD_OK;
    }

    // Tokens a sequence may attend to: T, plus the appended one.
    const long Tp = (long)T + ((o.flags & FD_FLAG_APPEND) ? 1 : 0);
    long gran = tile;
    if (paged && o.page_size > gran) gran = o.page_size;
    const long max_n = ceil_div(Tp, gran);
    long n;
    if (n_req > 0) {
        n = n_req < max_n ? n_req : max_n;
    } else {
        // About one workgroup per compute unit (measured best for streaming;
        // more, shorter splits only add partial traffic), but no split
        // shorter than min_chunk tokens (its partial write and
        // the merge must stay small against the chunk's KV bytes).  Paged
        // (ragged) batches get shorter chunks so the hardware scheduler can
        // balance sequences of very different lengths.
        const long units = (long)B * Hkv * head_blocks;
        const long target = std::max(1L, env_long("FD_TARGET_WGS", (long)cus));
        const long min_chunk = std::max(1L, env_long("FD_CHUNK_MIN", 512));
        n = ceil_div(target, units);
        const long cap = Tp / min_chunk > 1 ? Tp / min_chunk : 1;
        if (n > cap) n = cap;
        if (paged) {
            const long ragged_chunk = std::max(1L, env_long("FD_RAGGED_CHUNK", 1024));
            const long nr = ceil_div(Tp, ragged_chunk);
            if (n < nr) n = nr;
            // Workgroups go to the 8 XCDs round-robin by linear id, with the
            // split index fastest: a multiple of 8 splits spreads each
            // sequence's active (leading) splits evenly over the XCDs.
            n = ceil_div(n, 8) * 8;
        }
    }
    if (paged) {
        // a split stages its page ids on chip: at most kMaxSplitPages pages
        const long max_chunk = (long)fdk::kMaxSplitPages * o.page_size;
        const long n_min = ceil_div(Tp, max_chunk);
        if (n < n_min) n = n_min;
    }
    if (n < 1) n = 1;
    long chunk = ceil_div(ceil_div(Tp, n), gran) * gran;
    if (paged && chunk > (long)fdk::kMaxSplitPages * o.page_size)
        chunk = (long)fdk::kMaxSplitPages * o.page_size;
    n = ceil_div(Tp, chunk);

    p->n_splits = (int)n;
    p->chunk = (int)chunk;
    p->path = path;
    p->tile = tile;
    p->heads_per_block = hpb;
    p->head_blocks = head_blocks;
    p->grid[0] = (int)n;
    p->grid[1] = Hkv * head_blocks;
    p->grid[2] = B;
    p->block = 256;
    p->combine = n > 1;
    // The last workgroup of a group merges the splits itself when their
    // maxima and sums fit its LDS (n * heads <= 1024).  By default this is
    // chosen for small calls whose grid runs in about one round (at most two
    // workgroups per compute unit): there it saves the combine launch.  With
    // many rounds the per-workgroup publish latency costs more, and on large
    // calls the in-launch merge (its fences and the completing workgroup's
    // serial merge) costs more than the combine kernel.  Measured, wall time
    // per call: MHA f16 32k tokens x 32 heads (537 MB of K/V) 78.0 us
    // without any merge, 81.9 with the combine kernel, 83.6 fused; GQA 128k
    // bf16 (1.07 GB) 303.7 / 307.2 / 311.6; MHA with 4096 tokens (67 MB)
    // fused 18.3 vs 17.6 with the combine kernel, 2048 tokens (34 MB) 13.6
    // vs 15.8, the tiny fp32 case 9.3 vs 16.2.
    const double kv_call = 2.0 * B * Hkv * (double)Tp * D * elt;
    bool want_fused = (long)B * Hkv * head_blocks * n <= 2L * cus && kv_call <= kFusedMaxBytes;
    if (o.flags & FD_FLAG_FUSED_MERGE) want_fused = true;
    if (o.flags & FD_FLAG_COMBINE_KERNEL) want_fused = false;
    const long env_fused = env_long("FD_FUSED", -1);
    if (env_fused == 0 || env_fused == 1) want_fused = env_fused == 1;
    const long merge_heads = R < hpb ? R : hpb;
    p->fused = n > 1 && n * merge_heads <= fdk::kMergeMaxPairsHost && want_fused;
    if (n > 1) {
        const size_t parts = (size_t)B * Hkv * R * (size_t)n;
        const size_t counters = (size_t)B * Hkv * head_blocks * 2 * sizeof(unsigned long long);
        p->workspace_bytes = align256(counters) + align256(parts * D * sizeof(float)) +
                             2 * align256(parts * sizeof(float));
    }
    return FD_OK;
}

// FD_LOG=1: one line per planned call on stderr naming the kernel path and
// the plan that runs (the backend that ran is then on record).
bool log_enabled() {
    const char *e = std::getenv("FD_LOG");
    return e && e[0] == '1' && e[1] == '\0';
}

const char *path_name(int path) {
    switch (path) {
    case FD_PATH_VALU: return "valu";
    case FD_PATH_MFMA: return "mfma";
    case FD_PATH_PREFILL: return "query-tiled";
    default: return "?";
    }
}

void log_plan(const char *entry, int B, int Hq, int Hkv, int T, int D, int n_req, const fd_options_t &o,
              const fd_plan_t &p) {
    if (!log_enabled()) return;
    static const char *const dt[] = {"f32", "f16", "bf16"};
    const char *merge = p.n_splits <= 1 ? "none" : (p.stream || p.fused) ? "fused" : "combine-kernel";
    // 1: the order pass picks the split size on the device (at least `chunk`)
    const int on_device = p.path == FD_PATH_PREFILL &&
                          prefill_devchunk(prefill_ordered(o.page_size > 0, p.head_blocks, p.n_splits, B), n_req);
    std::fprintf(stderr,
                 "[fd] %s B=%d Hq=%d Hkv=%d T=%d D=%d dtype=%s n_queries=%d causal=%d paged=%d page_size=%d "
                 "n_splits_req=%d -> path=%s n_splits=%d chunk=%d chunk_on_device=%d grid=%dx%dx%d rows_per_wg=%d "
                 "head_blocks=%d merge=%s stream=%d workspace=%zu\n",
                 entry, B, Hq, Hkv, T, D, (o.dtype >= 0 && o.dtype <= 2) ? dt[o.dtype] : "?", (int)o.n_queries,
                 (int)o.causal, o.page_size > 0 ? 1 : 0, o.page_size > 0 ? (int)o.page_size : 0, n_req,
                 path_name(p.path), p.n_splits, p.chunk, on_device, p.grid[0], p.grid[1], p.grid[2],
                 p.heads_per_block, p.head_blocks, merge, p.stream, p.workspace_bytes);
}

struct Call {
    fd_options_t o;
    fd_plan_t p;
    fdk::SplitArgs s;
    fdk::CombineArgs c;
    fdk::PrefillArgs f;
};

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Everything fd_decode / fd_split / fd_combine check before launching.
// k_new / v_new: the appended token's rows (fd_append_decode), else nullptr.
fd_status_t prepare(const void *q, const void *k, const void *v, const int32_t *page_table,
                    const int32_t *seq_lens, float *out, float *lse, int B, int Hq, int Hkv,
                    int T, int D, float scale, int n_req, const fd_options_t *opt, bool need_inputs,
                    const void *k_new, const void *v_new, Call *c) {
    fd_status_t st = read_options(opt, &c->o);
    if (st != FD_OK) return st;
    const bool append = k_new != nullptr;
    if (append) {
        c->o.flags |= FD_FLAG_APPEND;
        if (!v_new) return fail(FD_ERR_INVALID_ARG, "k_new and v_new must be non-NULL");
        if (!aligned(k_new, 16) || !aligned(v_new, 16))
            return fail(FD_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
        if (k_new == k || v_new == v || k_new == v || v_new == k)
            return fail(FD_ERR_INVALID_ARG, "k_new and v_new must not be the caches");
    } else if (c->o.flags & FD_FLAG_APPEND) {
        return fail(FD_ERR_INVALID_ARG, "FD_FLAG_APPEND plans are run by fd_append_decode");
    }
    if (need_inputs) {
        if (!q || !k || !v) return fail(FD_ERR_INVALID_ARG, "q, k_cache and v_cache must be non-NULL");
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
            return fail(FD_ERR_INVALID_ARG, "q, k_cache and v_cache must be 16-byte aligned");
        if (!std::isfinite(scale)) return fail(FD_ERR_INVALID_ARG, "scale is not finite");
    }
    if (!out) return fail(FD_ERR_INVALID_ARG, "out must be non-NULL");
    if (!aligned(out, 16) || (lse && !aligned(lse, 4)))
        return fail(FD_ERR_INVALID_ARG, "out must be 16-byte and lse 4-byte aligned");
    if (seq_lens && !aligned(seq_lens, 4)) return fail(FD_ERR_INVALID_ARG, "seq_lens must be 4-byte aligned");
    // The page geometry in the options decides the plan; the split pass also
    // needs the table itself.
    const bool paged = c->o.page_size > 0;
    if (need_inputs && paged != (page_table != nullptr))
        return fail(FD_ERR_INVALID_ARG, "page_table and opt->page_size must be given together");
    if (page_table && !aligned(page_table, 4)) return fail(FD_ERR_INVALID_ARG, "page_table must be 4-byte aligned");
    st = make_plan(B, Hq, Hkv, T, D, n_req, c->o, paged, &c->p);
    if (st != FD_OK) return st;

    float *part_o = nullptr, *part_m = nullptr, *part_l = nullptr;
    unsigned long long *counters = nullptr;
    c->s.wg_clock = nullptr;
    if (c->p.stream) {
        if (!c->o.workspace)
            return fail(FD_ERR_WORKSPACE, "stream plan: a workspace of %zu bytes is required", c->p.workspace_bytes);
        if (c->o.workspace_bytes < c->p.workspace_bytes)
            return fail(FD_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", c->o.workspace_bytes,
                        c->p.workspace_bytes);
        if (!aligned(c->o.workspace, 256)) return fail(FD_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        const size_t rows = (size_t)B * Hkv * c->p.head_blocks;
        const size_t slots = (rows + (size_t)c->p.n_splits) * c->p.heads_per_block;
        char *w = static_cast<char *>(c->o.workspace);
        counters = reinterpret_cast<unsigned long long *>(w);
        w += align256(rows * 2 * sizeof(unsigned long long));
        part_o = reinterpret_cast<float *>(w);
        w += align256(slots * D * sizeof(float));
        part_m = reinterpret_cast<float *>(w);
        w += align256(slots * sizeof(float));
        part_l = reinterpret_cast<float *>(w);
        if (FD_WG_TIMING) {
            w += align256(slots * sizeof(float));
            c->s.wg_clock = reinterpret_cast<unsigned long long *>(w);
        }
    } else if (c->p.n_splits > 1 && c->p.path != FD_PATH_PREFILL) {
        if (!c->o.workspace)
            return fail(FD_ERR_WORKSPACE, "plan has %d splits: a workspace of %zu bytes is required",
                        c->p.n_splits, c->p.workspace_bytes);
        if (c->o.workspace_bytes < c->p.workspace_bytes)
            return fail(FD_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", c->o.workspace_bytes,
                        c->p.workspace_bytes);
        if (!aligned(c->o.workspace, 256)) return fail(FD_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        const size_t parts = (size_t)B * Hq * c->o.n_queries * (size_t)c->p.n_splits;
        char *w = static_cast<char *>(c->o.workspace);
        counters = reinterpret_cast<unsigned long long *>(w);
        w += align256((size_t)B * Hkv * c->p.head_blocks * 2 * sizeof(unsigned long long));
        part_o = reinterpret_cast<float *>(w);
        w += align256(parts * D * sizeof(float));
        part_m = reinterpret_cast<float *>(w);
        w += align256(parts * sizeof(float));
        part_l = reinterpret_cast<float *>(w);
    }

    fdk::SplitArgs &s = c->s;
    s.q = q; s.k = k; s.v = v;
    s.page_table = page_table;
    s.seq_lens = seq_lens;
    s.out = out; s.lse = lse;
    s.part_o = part_o; s.part_m = part_m; s.part_l = part_l;
    s.B = B; s.Hq = Hq; s.Hkv = Hkv; s.T = T; s.D = D; s.G = Hq / Hkv;
    s.nq = c->o.n_queries;
    s.R = s.nq * s.G;
    s.causal = c->o.causal;
    s.n_splits = c->p.n_splits;
    s.chunk = c->p.chunk;
    s.heads_per_block = c->p.heads_per_block;
    s.head_blocks = c->p.head_blocks;
    s.page_size = paged ? c->o.page_size : 1;
    s.page_shift = paged ? ilog2(c->o.page_size) : 0;
    s.max_pages = paged ? c->o.max_pages_per_seq : 0;
    s.num_pages = paged ? c->o.num_pages : 0;
    s.scale_log2 = (float)((double)scale * 1.4426950408889634074);
    s.fused = 0;
    s.epoch = 0;
    s.next_epoch = 0;
    s.counters = counters;
    s.stream = c->p.stream;
    s.stream_align = c->p.tile;
    {
        // MFMA kernel: ~256 tokens' worth per segment start, measured best on
        // the paged ragged batch (365.2 us against 369.8 us with none; 366.1
        // with 128, 364.9 with 384, 368.0 with 512, 370.5 with 1024; with 4
        // causal queries 378.6 against 389.8 us).  The VALU kernel's stream
        // mode measured 370.2 us with 256 against 368.7 with none.
        const long dflt = c->p.path == FD_PATH_MFMA ? 256 : 0;
        const long rc = std::max(0L, env_long("FD_STREAM_ROWCOST", dflt));
        s.stream_row_cost = (int)(ceil_div(std::min(rc, 1L << 20), (long)c->p.tile) * c->p.tile);
    }
    s.append = append ? 1 : 0;
    s.k_new = k_new;
    s.v_new = v_new;
    s.k_store = const_cast<void *>(k);
    s.v_store = const_cast<void *>(v);
    {
        const int merge_heads = s.R < c->p.heads_per_block ? s.R : c->p.heads_per_block;
        s.merge_cap = (int)(fdk::kMergeMaxPairsHost / merge_heads);
    }

    fdk::CombineArgs &cb = c->c;
    cb.part_o = part_o; cb.part_m = part_m; cb.part_l = part_l;
    cb.seq_lens = seq_lens;
    cb.out = out; cb.lse = lse;
    cb.B = B; cb.Hq = Hq; cb.T = T; cb.D = D;
    cb.Hkv = Hkv; cb.G = s.G; cb.nq = s.nq; cb.R = s.R;
    cb.n_splits = c->p.n_splits;
    cb.chunk = c->p.chunk;
    cb.dev_chunk = nullptr;
    cb.append = append ? 1 : 0;
    cb.causal = s.causal;
    // the query-tiled kernel's partials: many rows, few splits
    cb.per_wave = c->p.path == FD_PATH_PREFILL && env_long("FD_COMBINE_ROWS", 1) == 1 ? 1 : 0;

    fdk::PrefillArgs &f = c->f;
    f.q = q; f.k = k; f.v = v;
    f.page_table = page_table;
    f.seq_lens = seq_lens;
    f.out = out; f.lse = lse;
    f.B = B; f.nq = s.nq; f.Hq = Hq; f.Hkv = Hkv; f.T = T; f.D = D; f.G = s.G; f.R = s.R;
    f.row_tiles = c->p.path == FD_PATH_PREFILL ? c->p.head_blocks : 0;
    f.tile_rows = c->p.path == FD_PATH_PREFILL ? c->p.heads_per_block : 0;
    f.causal = s.causal;
    f.page_size = s.page_size; f.page_shift = s.page_shift; f.max_pages = s.max_pages; f.num_pages = s.num_pages;
    f.scale_log2 = s.scale_log2;
    f.vt = nullptr; f.vmax = nullptr; f.vexp = nullptr;
    // XCD-aware order.  Causal calls on a contiguous cache whose queries
    // cover at least half of it (row tiles from short to full length)
    // interleave each XCD's ranges in pairs (FD_PREFILL_PAIRS=0: one range
    // after another; 2: every causal call).  Measured: MHA f16 with 4096
    // causal queries over 4096 tokens 223 -> 211 us, B=2 x 2048 138 -> 125;
    // 512 causal queries over four paged 64k-token sequences 1393 -> 1860 us
    // and over B=8 x 8192 contiguous tokens 1132 -> 1150, hence the limits.
    const long pairs = env_long("FD_PREFILL_PAIRS", 1);
    const bool pair_ok = s.causal && (pairs == 2 || (pairs == 1 && !paged && 2L * s.nq >= T));
    f.xcd_map = env_long("FD_PREFILL_XCD", 1) == 1 ? (pair_ok ? 2 : 1) : 0;
    // paged pools below 4 GiB: 32-bit row offsets from the pool base
    f.pool32 = paged && (unsigned long long)c->o.num_pages * (unsigned long long)Hkv *
                                (unsigned long long)c->o.page_size * (unsigned long long)D * 2ull <
                            (1ull << 32) &&
               env_long("FD_PREFILL_POOL32", 1) == 1;
    f.vt_tiles = (int)ceil_div(T, fdk::kPrefillTokens);
    f.vmax_chunks = (int)ceil_div(T, fdk::kVconvChunk);
    f.n_splits = c->p.path == FD_PATH_PREFILL ? c->p.n_splits : 1;
    f.chunk = c->p.chunk;
    f.part_o = f.part_m = f.part_l = nullptr;
    f.order = nullptr;
    f.dev_chunk = nullptr;
    f.slots = 0;
    if (c->p.path == FD_PATH_PREFILL && c->p.workspace_bytes > 0) {
        if (!c->o.workspace)
            return fail(FD_ERR_WORKSPACE, "query-tiled plan: a workspace of %zu bytes is required",
                        c->p.workspace_bytes);
        if (c->o.workspace_bytes < c->p.workspace_bytes)
            return fail(FD_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", c->o.workspace_bytes,
                        c->p.workspace_bytes);
        if (!aligned(c->o.workspace, 256)) return fail(FD_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        // converted V (bf16), then the split partials, then the column order
        const bool ordered = prefill_ordered(paged, c->p.head_blocks, c->p.n_splits, B);
        const size_t order_bytes = ordered ? fdk::prefill_order_bytes(B, c->p.n_splits) : 0;
        const size_t vt_bytes =
            c->p.workspace_bytes - fdk::prefill_part_bytes(B, Hkv, s.R, D, c->p.n_splits) - order_bytes;
        char *w = static_cast<char *>(c->o.workspace);
        if (ordered) {
            f.order = reinterpret_cast<uint32_t *>(w + (c->p.workspace_bytes - order_bytes));
            if (prefill_devchunk(ordered, n_req)) {
                // after the order entries; the workgroups resident at once:
                // three per CU for the paged 64-row instance with V read as
                // given, two for the others
                f.dev_chunk = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(f.order) +
                                                          align256((size_t)B * c->p.n_splits * 4));
                int cus = c->o.num_cus;
                if (cus == 0) {
                    const fd_status_t cst = device_cus(&cus);
                    if (cst != FD_OK) return cst;
                }
                const bool three = f.tile_rows == fdk::kPrefillSmallRows && vt_bytes == 0;
                f.slots = (three ? 3 : 2) * cus;
                cb.dev_chunk = f.dev_chunk;
            }
        }
        if (vt_bytes > 0) {
            const size_t sl = (size_t)B * Hkv;
            f.vexp = reinterpret_cast<int32_t *>(w);
            f.vmax = reinterpret_cast<uint32_t *>(w + align256(sl * 4));
            f.vt = reinterpret_cast<uint16_t *>(w + align256(sl * 4) + align256(sl * f.vmax_chunks * 4));
        }
        if (c->p.n_splits > 1) {
            const size_t parts = (size_t)B * Hkv * s.R * (size_t)c->p.n_splits;
            w += vt_bytes;
            f.part_o = reinterpret_cast<float *>(w);
            w += align256(parts * D * sizeof(float));
            f.part_m = reinterpret_cast<float *>(w);
            w += align256(parts * sizeof(float));
            f.part_l = reinterpret_cast<float *>(w);
            cb.part_o = f.part_o;
            cb.part_m = f.part_m;
            cb.part_l = f.part_l;
        }
    }
    return FD_OK;
}

// Epochs of fused calls.  A fresh epoch is distinct from every other one
// this process hands out (never 0 and never all ones, the values a cleared
// or poisoned word reads), so counters left by any other call are stale.
unsigned fresh_epoch() {
    static std::atomic<unsigned> epoch{0x5eed0000u};
    unsigned e;
    do { e = epoch.fetch_add(1, std::memory_order_relaxed) + 1; } while (e == 0 || e == ~0u);
    return e;
}

// The epoch each recent workspace's counters were left at by its last fused
// call: the next call on that workspace uses it, so its arrivals take the
// one-fetch-add path.  A workspace not found here (first use, or evicted)
// gets a fresh epoch and counts once through the exchange loop; results do
// not depend on this table, only the cost of the count does.
struct EpochTable {
    static constexpr int kSlots = 64;
    std::mutex mu;
    const void *ws[kSlots] = {};
    unsigned left[kSlots] = {};
    int victim = 0;

    // (epoch for this call, epoch its completing workgroups leave behind)
    void take(const void *w, unsigned *cur, unsigned *next) {
        std::lock_guard<std::mutex> g(mu);
        *next = fresh_epoch();
        for (int i = 0; i < kSlots; ++i)
            if (ws[i] == w) {
                *cur = left[i];
                left[i] = *next;
                return;
            }
        *cur = fresh_epoch();
        ws[victim] = w;
        left[victim] = *next;
        victim = (victim + 1) % kSlots;
    }

    // A launch captured into a graph: it runs later, once per replay, with
    // the arguments fixed now.  It gets one fresh epoch as both its own and
    // the one it leaves, so each replay leaves the counters tagged for the
    // next replay (the first replay counts through the slow word).  Eager
    // calls after the replays find the tag here.
    void take_captured(const void *w, unsigned *cur, unsigned *next) {
        std::lock_guard<std::mutex> g(mu);
        *cur = *next = fresh_epoch();
        for (int i = 0; i < kSlots; ++i)
            if (ws[i] == w) {
                left[i] = *cur;
                return;
            }
        ws[victim] = w;
        left[victim] = *cur;
        victim = (victim + 1) % kSlots;
    }

    // the launch failed: the counters were not touched
    void forget(const void *w) {
        std::lock_guard<std::mutex> g(mu);
        for (int i = 0; i < kSlots; ++i)
            if (ws[i] == w) ws[i] = nullptr;
    }
};

EpochTable g_epochs;

fd_status_t run_split(Call &c, bool fused) {
    if (c.p.path == FD_PATH_PREFILL) {
        const hipError_t e = fdk::launch_prefill(c.f, c.o.dtype, static_cast<hipStream_t>(c.o.stream));
        if (e != hipSuccess) return hip_fail(e, "launching the query-tiled kernel");
        return FD_OK;
    }
    fused = fused || c.p.stream;            // stream mode always merges in the launch
    c.s.fused = fused ? 1 : 0;
    c.s.epoch = c.s.next_epoch = 0;
    const hipStream_t stream = static_cast<hipStream_t>(c.o.stream);
    if (fused) {
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        const hipError_t ce = hipStreamIsCapturing(stream, &cap);
        if (ce != hipSuccess) return hip_fail(ce, "hipStreamIsCapturing");
        if (cap == hipStreamCaptureStatusActive)
            g_epochs.take_captured(c.s.counters, &c.s.epoch, &c.s.next_epoch);
        else
            g_epochs.take(c.s.counters, &c.s.epoch, &c.s.next_epoch);
    }
    const hipError_t e = c.p.path == FD_PATH_MFMA ? fdk::launch_split_mfma(c.s, c.o.dtype, stream)
                                                  : fdk::launch_split_valu(c.s, c.o.dtype, stream);
    if (e != hipSuccess) {
        if (fused) g_epochs.forget(c.s.counters);
        return hip_fail(e, "launching the split kernel");
    }
    return FD_OK;
}

fd_status_t run_combine(const Call &c) {
    if (c.p.n_splits <= 1 || c.p.stream) return FD_OK;
    const hipError_t e = fdk::launch_combine(c.c, static_cast<hipStream_t>(c.o.stream));
    if (e != hipSuccess) return hip_fail(e, "launching the combine kernel");
    return FD_OK;
}

}  // namespace

namespace fdk {

fd_status_t scratch_plan(const void *q, const void *k_cache, const void *v_cache, const int32_t *page_table,
                         const int32_t *seq_lens, float *out, float *lse, int B, int Hq, int Hkv, int T, int D,
                         float scale, int n_splits, const fd_options_t *opt, size_t scratch_bytes) {
    fd_options_t o;
    fd_status_t st = read_options(opt, &o);
    if (st != FD_OK) return st;
    if (o.workspace || o.workspace_bytes)
        return fail(FD_ERR_INVALID_ARG,
                    "fd_decode_noalloc uses the library's own scratch: opt->workspace must be NULL and "
                    "opt->workspace_bytes 0");
    fd_plan_t p;
    st = make_plan(B, Hq, Hkv, T, D, n_splits, o, o.page_size > 0, &p);
    if (st != FD_OK) return st;
    if (p.workspace_bytes > scratch_bytes)
        return fail(FD_ERR_WORKSPACE,
                    "this call needs %zu bytes of scratch, more than the %zu-byte static scratch of "
                    "fd_decode_noalloc holds; call fd_decode with a caller-owned workspace instead",
                    p.workspace_bytes, scratch_bytes);
    // every other check of fd_decode, with a stand-in workspace address (the
    // host never dereferences it)
    o.workspace = reinterpret_cast<void *>(uintptr_t(256));
    o.workspace_bytes = scratch_bytes;
    Call c;
    return prepare(q, k_cache, v_cache, page_table, seq_lens, out, lse, B, Hq, Hkv, T, D, scale, n_splits, &o, true,
                   nullptr, nullptr, &c);
}

fd_status_t decode_with_scratch(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *page_table, const int32_t *seq_lens, float *out, float *lse,
                                int B, int Hq, int Hkv, int T, int D, float scale, int n_splits,
                                const fd_options_t *opt, void *scratch, size_t scratch_bytes) {
    fd_options_t o;
    fd_status_t st = read_options(opt, &o);
    if (st != FD_OK) return st;
    o.workspace = scratch;
    o.workspace_bytes = scratch_bytes;
    Call c;
    st = prepare(q, k_cache, v_cache, page_table, seq_lens, out, lse, B, Hq, Hkv, T, D, scale, n_splits, &o, true,
                 nullptr, nullptr, &c);
    if (st != FD_OK) return st;
    log_plan("fd_decode_noalloc", B, Hq, Hkv, T, D, n_splits, c.o, c.p);
    const bool fused = c.p.fused != 0;
    st = run_split(c, fused);
    if (st != FD_OK || fused) return st;
    return run_combine(c);
}

fd_status_t hip_error(hipError_t e, const char *what) { return hip_fail(e, what); }

fd_status_t error(fd_status_t st, const char *msg) { return fail(st, "%s", msg); }

}  // namespace fdk

extern "C" {

void fd_options_init(fd_options_t *opt) {
    if (!opt) return;
    std::memset(opt, 0, sizeof *opt);
    opt->struct_size = sizeof *opt;
    opt->dtype = FD_BF16;
    opt->path = FD_PATH_AUTO;
    opt->n_queries = 1;
}

fd_status_t fd_plan(int B, int Hq, int Hkv, int T, int D, int n_splits, const fd_options_t *opt,
                    fd_plan_t *plan) {
    if (!plan) return fail(FD_ERR_INVALID_ARG, "plan pointer is NULL");
    fd_options_t o;
    fd_status_t st = read_options(opt, &o);
    if (st != FD_OK) return st;
    st = make_plan(B, Hq, Hkv, T, D, n_splits, o, o.page_size > 0, plan);
    if (st == FD_OK) log_plan("fd_plan", B, Hq, Hkv, T, D, n_splits, o, *plan);
    return st;
}

size_t fd_workspace_bytes(int B, int Hq, int Hkv, int T, int D, int n_splits, const fd_options_t *opt) {
    fd_plan_t p;
    if (fd_plan(B, Hq, Hkv, T, D, n_splits, opt, &p) != FD_OK) return 0;
    return p.workspace_bytes;
}

fd_status_t fd_decode(const void *q, const void *k_cache, const void *v_cache, const int32_t *page_table,
                      const int32_t *seq_lens, float *out, float *lse, int B, int Hq, int Hkv, int T, int D,
                      float scale, int n_splits, const fd_options_t *opt) {
    Call c;
    fd_status_t st = prepare(q, k_cache, v_cache, page_table, seq_lens, out, lse, B, Hq, Hkv, T, D, scale,
                             n_splits, opt, true, nullptr, nullptr, &c);
    if (st != FD_OK) return st;
    log_plan("fd_decode", B, Hq, Hkv, T, D, n_splits, c.o, c.p);
    const bool fused = c.p.fused != 0;
    st = run_split(c, fused);
    if (st != FD_OK || fused) return st;
    return run_combine(c);
}

fd_status_t fd_append_decode(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                             const int32_t *page_table, const int32_t *seq_lens, float *out, float *lse, int B,
                             int Hq, int Hkv, int T, int D, float scale, int n_splits, const fd_options_t *opt) {
    Call c;
    if (!k_new) return fail(FD_ERR_INVALID_ARG, "k_new and v_new must be non-NULL");
    fd_status_t st = prepare(q, k_cache, v_cache, page_table, seq_lens, out, lse, B, Hq, Hkv, T, D, scale,
                             n_splits, opt, true, k_new, v_new, &c);
    if (st != FD_OK) return st;
    log_plan("fd_append_decode", B, Hq, Hkv, T, D, n_splits, c.o, c.p);
    const bool fused = c.p.fused != 0;
    st = run_split(c, fused);
    if (st != FD_OK || fused) return st;
    return run_combine(c);
}

fd_status_t fd_split(const void *q, const void *k_cache, const void *v_cache, const int32_t *page_table,
                     const int32_t *seq_lens, float *out, float *lse, int B, int Hq, int Hkv, int T, int D,
                     float scale, int n_splits, const fd_options_t *opt) {
    Call c;
    fd_status_t st = prepare(q, k_cache, v_cache, page_table, seq_lens, out, lse, B, Hq, Hkv, T, D, scale,
                             n_splits, opt, true, nullptr, nullptr, &c);
    if (st != FD_OK) return st;
    log_plan("fd_split", B, Hq, Hkv, T, D, n_splits, c.o, c.p);
    return run_split(c, false);
}

fd_status_t fd_combine(const int32_t *seq_lens, float *out, float *lse, int B, int Hq, int Hkv, int T, int D,
                       int n_splits, const fd_options_t *opt) {
    Call c;
    fd_status_t st = prepare(nullptr, nullptr, nullptr, nullptr, seq_lens, out, lse, B, Hq, Hkv, T, D, 1.0f,
                             n_splits, opt, false, nullptr, nullptr, &c);
    if (st != FD_OK) return st;
    log_plan("fd_combine", B, Hq, Hkv, T, D, n_splits, c.o, c.p);
    return run_combine(c);
}

const char *fd_status_string(fd_status_t status) {
    switch (status) {
    case FD_OK: return "FD_OK";
    case FD_ERR_INVALID_ARG: return "FD_ERR_INVALID_ARG: invalid argument";
    case FD_ERR_UNSUPPORTED: return "FD_ERR_UNSUPPORTED: no kernel for these arguments";
    case FD_ERR_WORKSPACE: return "FD_ERR_WORKSPACE: workspace missing or too small";
    case FD_ERR_HIP: return "FD_ERR_HIP: HIP runtime error";
    default: return "unknown fd_status_t";
    }
}

const char *fd_last_error(void) { return g_err; }

}  // extern "C"
