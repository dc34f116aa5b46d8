/*
 * fd.h -- C ABI of libfd: split-KV ("flash decoding") single-query decode
 * attention for AMD Instinct MI355X (gfx950).
 *
 * The operation (tinyvolt "Kernel visualization: Flash Decoding", opening
 * section and its split / combine kernels; zenaique explainer, "What decode
 * looks like"): for every batch row b and query head h, with kv head
 * j = h / (Hq / Hkv) and valid length T_b,
 *
 *     out[b,h,:] = softmax_t( scale * q[b,h,:] . K[b,j,t,:] ) @ V[b,j,t,:]
 *     lse[b,h]   = ln sum_t exp( scale * q[b,h,:] . K[b,j,t,:] )
 *
 * computed by splitting the KV axis into chunks: a split pass runs an
 * online softmax over each chunk and keeps an unnormalised partial with its
 * running max and sum; a combine pass aligns the partials to the global max
 * and divides once.  The result equals the whole softmax up to fp32
 * rounding order (zenaique explainer, interview answer on exactness).
 *
 * Conventions shared by every entry point:
 *   - All tensor arguments are DEVICE pointers on the current HIP device,
 *     contiguous, row-major.  The caller allocates and owns every buffer,
 *     including the workspace (fd_decode_noalloc uses a static scratch of
 *     the library instead); the library keeps no pointer after a call
 *     returns and allocates no device memory.
 *   - q: [B, Hq, D]; contiguous caches: [B, Hkv, T, D]; paged pools:
 *     [num_pages, Hkv, page_size, D] with page_table [B, max_pages_per_seq]
 *     int32 (token t of sequence b is row t % page_size of page
 *     page_table[b][t / page_size]); seq_lens [B] int32 with 0 <= T_b <= T.
 *     q, K and V share one storage dtype (fd_options_t.dtype); q, K, V and
 *     out must be 16-byte aligned.  out is [B, Hq, D] fp32, lse [B, Hq] fp32 (natural
 *     log; may be NULL).  A sequence with T_b = 0 yields out = 0 and
 *     lse = -inf.
 *   - Several queries per sequence (fd_options_t.n_queries = n_q > 1; the
 *     dupenodi guide "FlashDecoding and split-KV" has decode run one query
 *     or a small batch of queries against the cache): q is [B, n_q, Hq, D],
 *     out [B, n_q, Hq, D], lse [B, n_q, Hq].  Every query of a sequence
 *     reads the same K / V once per pass; query i attends to the first T_b
 *     tokens, or with fd_options_t.causal to the first T_b - (n_q - 1 - i)
 *     (the queries are the sequence's last n_q cached tokens, as in
 *     verifying a draft); a query with no token yields out = 0, lse = -inf.
 *     Up to 16 queries run on the split-KV kernels (every query row of a kv
 *     head shares one read of K / V), as long as a kv head has at most 16
 *     query rows (n_q * G) or the inputs are fp32;
 *     more queries (the
 *     prefill phase: the dupenodi guide, "Concept", has prefill attend with
 *     the whole block of prompt queries), or more rows, run on a query-tiled
 *     kernel: one workgroup per 128 query rows of a (sequence, kv head) and
 *     KV split (FD_PATH_PREFILL; f16 / bf16 only).  The planner splits the
 *     KV axis only when the row tiles alone leave the device short of
 *     workgroups (few queries over a long cache, or a ragged batch, planned
 *     for its longest sequence T); the splits'
 *     partials are then merged by the combine kernel, as in decode, and
 *     n_splits > 0 asks for that many splits.  The workspace
 *     (fd_plan_t.workspace_bytes) holds, for bf16 with at least 1024 query
 *     rows per kv head, V converted by two passes ahead of the kernel to f16
 *     under a power-of-two scale per (sequence, kv head) -- exact for every
 *     value above 2^-28 of the slice's largest |V|, so the value product
 *     runs on f16 with one probability product; about the size of the V
 *     slices (fewer rows keep bf16 V and split the probabilities into two
 *     bf16 parts instead) -- followed, with several splits, by
 *     the partials [B, Hkv, n_q * G, n_splits, D] and two
 *     [B, Hkv, n_q * G, n_splits] rows.  One-split f16 calls need none.
 *   - A few FD_* environment variables, read when a call is planned, switch
 *     planner and kernel choices for measurement; every setting computes the
 *     same attention (within the tolerances above) and the defaults are the
 *     measured choices.
 *   - Calls are stream-ordered on fd_options_t.stream and never synchronise;
 *     a fault inside a kernel surfaces at the caller's next synchronisation.
 *   - Arguments are validated on the host before any launch.  Every call
 *     returns an fd_status_t; no exception crosses the ABI and the library
 *     never exits the process.  fd_last_error() returns this thread's
 *     message for the last failing call.
 *   - Argument checking and planning are thread-safe.  Concurrent calls
 *     that share one workspace must be ordered by the caller's streams.
 */
#ifndef FD_H
#define FD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FD_F32 = 0,
    FD_F16 = 1,
    FD_BF16 = 2
} fd_dtype_t;

typedef enum {
    FD_OK = 0,
    FD_ERR_INVALID_ARG = 1,   /* a pointer, size or option is invalid        */
    FD_ERR_UNSUPPORTED = 2,   /* valid, but no kernel instance (e.g. D=96)    */
    FD_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required   */
    FD_ERR_HIP = 4            /* a HIP runtime call failed (see fd_last_error) */
} fd_status_t;

typedef enum {
    FD_PATH_AUTO = -1,        /* the planner chooses                          */
    FD_PATH_VALU = 0,         /* vector-ALU dot products and reductions       */
    FD_PATH_MFMA = 1,         /* matrix-core path (f16/bf16 only)             */
    FD_PATH_PREFILL = 2       /* query-tiled matrix-core kernel for many      */
                              /* queries per sequence (f16/bf16; no split)    */
} fd_path_t;

/* fd_options_t.flags.  By default fd_decode merges the splits inside the
 * split launch (the last workgroup of each kv head combines its group; the
 * partials are ordered by a release fence before each arrival and an
 * acquire fence in the completing workgroup) for small calls -- at most 48
 * MiB of K/V, counted at T for every sequence -- whose grid runs in about
 * one round of workgroups, and launches the combine kernel otherwise;
 * stream mode (paged batches, automatic split count) always merges in the
 * launch.  These flags force one or the other. */
#define FD_FLAG_FUSED_MERGE 0x1
#define FD_FLAG_COMBINE_KERNEL 0x2
/* Plan for fd_append_decode: every sequence attends to one more token than
 * it has cached (plans cover T + 1 tokens).  Pass it to fd_plan /
 * fd_workspace_bytes to size the workspace of an append call;
 * fd_append_decode sets it itself, and fd_decode / fd_split / fd_combine
 * reject it. */
#define FD_FLAG_APPEND 0x4

/* Options of a call.  Initialise with fd_options_init() and then set the
 * fields you need; struct_size versions the layout. */
typedef struct fd_options {
    uint32_t struct_size;       /* sizeof(fd_options_t) of the caller         */
    int32_t dtype;              /* fd_dtype_t of q, K and V                    */
    int32_t page_size;          /* > 0 selects the paged layout (page_table   */
                                /* required): tokens per page, power of two   */
    int32_t max_pages_per_seq;  /* paged only: row stride of page_table       */
    int32_t num_pages;          /* paged only: pool size; page ids outside    */
                                /* [0, num_pages) read as empty tokens        */
    int32_t num_cus;            /* compute units to plan for; 0 = ask device  */
    int32_t path;               /* fd_path_t; FD_PATH_AUTO by default          */
    int32_t flags;              /* FD_FLAG_* bits; 0 by default               */
    void *workspace;            /* device buffer for the split partials        */
    size_t workspace_bytes;     /* its size in bytes                          */
    void *stream;               /* hipStream_t to launch on; NULL = null stream */
    int32_t n_queries;          /* queries per sequence, 1 .. 65536 (0 = 1);  */
                                /* > 1 gives q / out an n_q axis (see below); */
                                /* > 16 (or > 32 query rows per kv head,     */
                                /* f16 / bf16) runs the query-tiled kernel   */
    int32_t causal;             /* with n_queries > 1: 1 = query i sees the   */
                                /* first T_b - (n_queries - 1 - i) tokens     */
} fd_options_t;

/* What a call with these arguments will launch (see fd_plan).  Paged calls
 * (opt->page_size > 0) are planned as ragged batches: with the automatic
 * split count (and B <= 2048) in stream mode, else with short chunks, so
 * sequences of very different lengths spread evenly over the device. */
typedef struct fd_plan {
    int32_t n_splits;           /* effective number of KV splits              */
    int32_t chunk;              /* tokens per split (last one may be shorter) */
    int32_t path;               /* fd_path_t that runs                        */
    int32_t tile;               /* tokens one workgroup consumes per step     */
    int32_t heads_per_block;    /* query heads of one kv group per workgroup  */
                                /* (query-tiled plans: rows per row tile)     */
    int32_t head_blocks;        /* workgroups across one kv head's group      */
                                /* (query-tiled plans: row tiles)             */
    int32_t grid[3];            /* split-kernel grid (x: split, y: kv head *  */
                                /* head_blocks, z: batch; query-tiled plans:  */
                                /* x: row tiles * splits, y: kv head, z: batch) */
    int32_t block;              /* threads per split workgroup                */
    int32_t combine;            /* 1 if the splits are merged (n_splits > 1)   */
    int32_t fused;              /* 1 if fd_decode merges them inside the split */
                                /* launch (its last workgroup per kv head);   */
                                /* 0: fd_decode launches the combine kernel   */
    int32_t stream;             /* 1: balanced stream mode (paged, automatic  */
                                /* split count): grid[0] workgroups each take */
                                /* an equal share of all rows' tokens; chunk  */
                                /* is 0 and n_splits = grid[0]; the merge is  */
                                /* always inside the split launch             */
    int32_t reserved;
    size_t workspace_bytes;     /* workspace this call needs (0 for one split,  */
                                /* except bf16 query-tiled plans that convert V) */
} fd_plan_t;

/* Fill *opt with defaults: dtype bf16, contiguous cache, automatic path,
 * no workspace, null stream. */
void fd_options_init(fd_options_t *opt);

/*
 * Choose the split count and kernel for a call (host only; no GPU work).
 * n_splits > 0 asks for that many splits (capped so no split is empty when
 * every sequence has length T, and raised for paged layouts so one split
 * covers at most 2048 pages); n_splits = 0 lets the planner size the grid
 * to the device: enough (batch, kv head, split) workgroups to cover every
 * compute unit, with each split long enough to amortise its partial write
 * (the occupancy argument of the zenaique explainer, "Why decode breaks
 * FlashAttention v2").  num_cus = 0 in *opt queries the current device.
 * Returns FD_OK and fills *plan, or an error status.
 */
fd_status_t fd_plan(int B, int Hq, int Hkv, int T, int D, int n_splits,
                    const fd_options_t *opt, fd_plan_t *plan);

/* Workspace bytes fd_decode needs for these arguments (0 when the plan has
 * one split, or when the arguments are invalid -- check fd_plan then). */
size_t fd_workspace_bytes(int B, int Hq, int Hkv, int T, int D, int n_splits,
                          const fd_options_t *opt);

/*
 * Decode attention: the split pass and, when the plan has more than one
 * split, the merge of the splits, on opt->stream.  With plan.fused the
 * merge runs inside the split launch (the last workgroup of each kv head
 * combines its group's splits), so one kernel is launched; otherwise the
 * combine kernel follows.
 *   q, k_cache, v_cache : device inputs in opt->dtype (layouts above).
 *   page_table          : NULL for contiguous caches; else [B, max_pages].
 *   seq_lens            : NULL = every sequence has length T; else [B].
 *   out, lse            : device outputs, fp32; lse may be NULL.
 *   T                   : cache length, or the largest T_b for ragged input.
 *   scale               : multiplies q.k before the softmax (finite).
 *   n_splits            : 0 = automatic, else the requested split count.
 * The workspace (opt->workspace, >= fd_workspace_bytes, 256-byte aligned)
 * holds two arrival counter words per (batch, kv head, head block), the partials
 * [B, Hq, n_splits, D] and two [B, Hq, n_splits] rows (a stream plan: one
 * partial slot per (row + workgroup) pair instead).  Its contents before
 * the call do not matter: counters carry a per-call tag, so values left by
 * any other call are ignored (a fused call leaves its counters tagged for
 * the next call on the same workspace, which then counts arrivals with one
 * atomic add each; anything else is counted once through a slower exchange
 * loop).  The completing workgroup of each group resets both counter words,
 * so a call captured into a HIP graph (detected with hipStreamIsCapturing)
 * counts correctly on every replay.  Calls that share a workspace must not
 * overlap in time.
 *
 * FD_LOG=1 in the environment prints one line per planned call on stderr:
 * the entry point, the shape, and the plan that runs (kernel path, split
 * count and chunk, grid, merge form, stream mode, workspace bytes).
 */
fd_status_t fd_decode(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *page_table, const int32_t *seq_lens,
                      float *out, float *lse,
                      int B, int Hq, int Hkv, int T, int D, float scale,
                      int n_splits, const fd_options_t *opt);

/*
 * Fused append-KV decode step (dupenodi guide "FlashDecoding and split-KV",
 * "Walking through it": serving stacks pair split-KV decode with fused
 * append-KV paths).  In one pass over the cache, for every sequence b with
 * T_b = seq_lens[b] cached tokens (T when seq_lens is NULL):
 *   - the new token's rows k_new[b, j, :] and v_new[b, j, :] (every kv
 *     head j) are stored as token T_b of the cache: row T_b of a contiguous
 *     cache, or row T_b % page_size of page page_table[b, T_b / page_size];
 *   - out / lse are decode attention over tokens 0 .. T_b, the new one
 *     included (read from k_new / v_new, not from the cache).
 *   k_new, v_new : device, [B, Hkv, D] in opt->dtype, 16-byte aligned; they
 *                  must not overlap the caches.
 *   k_cache, v_cache : written at the new token's slot only.  A sequence
 *                  whose cache is full (T_b = T; paged: no table column
 *                  T_b / page_size, or a column naming no pool page) stores
 *                  nothing but still attends to its new token.
 *   seq_lens     : lengths before the append; the library does not update
 *                  them (the caller adds one for the next step).
 * Everything else as fd_decode; the workspace is sized by fd_workspace_bytes
 * with FD_FLAG_APPEND in opt->flags.
 */
fd_status_t fd_append_decode(const void *q, const void *k_new, const void *v_new,
                             void *k_cache, void *v_cache,
                             const int32_t *page_table, const int32_t *seq_lens,
                             float *out, float *lse,
                             int B, int Hq, int Hkv, int T, int D, float scale,
                             int n_splits, const fd_options_t *opt);

/*
 * The split pass alone (tinyvolt, "Visualizing operations in a single
 * block"): one workgroup per (batch, kv head, split) streams its chunk of K
 * and V and writes the unnormalised partial, its max and its sum to the
 * workspace.  With a one-split plan it normalises and writes out / lse
 * itself; a stream plan always merges inside this launch, so its out / lse
 * are final.  Same arguments as fd_decode.
 */
fd_status_t fd_split(const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *page_table, const int32_t *seq_lens,
                     float *out, float *lse,
                     int B, int Hq, int Hkv, int T, int D, float scale,
                     int n_splits, const fd_options_t *opt);

/*
 * The combine pass alone (tinyvolt, "Combine kernel"): one workgroup per
 * (batch, query head) merges the partials fd_split left in the workspace by
 * log-sum-exp and writes out / lse.  Must follow fd_split with the same
 * B, Hq, Hkv, T, D, n_splits, seq_lens and options.  A no-op (FD_OK) when
 * the plan has one split or is a stream plan (whose split launch merges).
 */
fd_status_t fd_combine(const int32_t *seq_lens, float *out, float *lse,
                       int B, int Hq, int Hkv, int T, int D, int n_splits,
                       const fd_options_t *opt);

/*
 * fd_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same call, whose workspace is a static device array of the library
 * (FD_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends) instead of
 * a caller-owned buffer.  Allocates nothing (no hipMalloc, no allocating
 * library routine); the caller still passes inputs and outputs.
 *   opt->workspace must be NULL and opt->workspace_bytes 0 (else
 *   FD_ERR_INVALID_ARG).  A call whose plan needs more workspace than the
 *   scratch holds (fd_workspace_bytes > FD_NOALLOC_SCRATCH_BYTES) fails with
 *   FD_ERR_WORKSPACE before any device work; fd_decode with a caller-owned
 *   workspace serves it.
 *   The scratch keeps the last call's contents; nothing in it must start at
 *   zero (counters carry per-call tags).  Every call on one GPU uses that
 *   GPU's one array, so calls that overlap in time on one GPU (other
 *   streams, other threads) race and give wrong results: order them.
 * Results are those of fd_decode with the same arguments.
 */
#define FD_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

fd_status_t fd_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *page_table, const int32_t *seq_lens,
                              float *out, float *lse,
                              int B, int Hq, int Hkv, int T, int D, float scale,
                              int n_splits, const fd_options_t *opt);

/* Static text for a status code. */
const char *fd_status_string(fd_status_t status);

/* This thread's message for the last call that did not return FD_OK
 * ("" if none).  Valid until the thread's next failing call. */
const char *fd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FD_H */
