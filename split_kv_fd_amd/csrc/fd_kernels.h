// Internal interface between the host library (fd_api.cpp) and the HIP
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/fd.h"

// Tokens each row of a wave takes per step in the VALU kernel (G <= 2).
#ifndef FD_VALU_U
#define FD_VALU_U 4
#endif
// 1: stream K/V with non-temporal loads (each byte is read once; keeping
// it out of the caches measured 13-19% faster on MI355X).
#ifndef FD_NT_LOADS
#define FD_NT_LOADS 1
#endif

namespace fdk {

// Page ids one split workgroup stages in LDS (paged layout): a paged split
// covers at most kMaxSplitPages pages, so the planner keeps paged chunks at
// or below kMaxSplitPages * page_size tokens.
constexpr int kMaxSplitPages = 2048;
// Largest heads x splits a fused merge handles (its LDS arrays).
constexpr long kMergeMaxPairsHost = 1024;

// Everything one split launch needs.  Passed by value as the kernel argument.
struct SplitArgs {
    const void *q;
    const void *k;
    const void *v;
    const int32_t *page_table;   // nullptr: contiguous cache
    const int32_t *seq_lens;     // nullptr: every sequence has length T
    float *out;                  // written directly when n_splits == 1
    float *lse;                  // may be nullptr
    float *part_o;               // [B, Hq, n_splits, D] unnormalised
    float *part_m;               // [B, Hq, n_splits] running max, log2 units
    float *part_l;               // [B, Hq, n_splits] running sum
    int B, Hq, Hkv, T, D, G;     // G = Hq / Hkv
    // Query rows of one kv head: R = nq * G, row r = (query r / G, head
    // r % G of the group).  Head blocks tile the rows; partials are indexed
    // by row: [B, Hkv, R, n_splits].
    int nq, R;
    int causal;                  // query i sees the first T_b - (nq - 1 - i) tokens
    int n_splits, chunk;
    int heads_per_block, head_blocks;
    int page_size, page_shift, max_pages, num_pages;
    float scale_log2;            // scale * log2(e): logits in base-2 units
    int fused;                   // last workgroup of a group merges its splits
    unsigned epoch;              // per-call tag of the arrival counters
    unsigned next_epoch;         // tag the completing workgroup leaves for the next call
    unsigned long long *counters;  // arrival counters, two words per group (row)
    // Stream mode (ragged batches): rows padded to stream_align tokens and
    // laid end to end, one equal range per workgroup (gridDim.x of them).
    int stream;
    int stream_align;
    int stream_row_cost;         // stream positions before each row's tokens (multiple of stream_align)
    int merge_cap;               // most segments one row may have (fused merge)
    // Append (fused append-KV): the new token's rows k_new / v_new [B, Hkv,
    // D] are token T_b = seq_lens[b] of each sequence, which then has T_b + 1
    // tokens; the workgroup that covers it also stores them into the caches.
    int append;
    const void *k_new;
    const void *v_new;
    void *k_store;               // the caches again, writable
    void *v_store;
    // Measurement builds (FD_WG_TIMING=1) only: kWgClockSlots real-time
    // clock marks per stream-mode workgroup; nullptr otherwise.
    unsigned long long *wg_clock;
};

#ifndef FD_WG_TIMING
#define FD_WG_TIMING 0
#endif
// Stream-mode clock marks of a measurement build, per workgroup: 0 start,
// 1 lengths scanned, then for each of the first three segments i: 2+4i
// start, 3+4i page ids staged, 4+4i tokens streamed, 5+4i result
// published; 14 deferred arrivals start, 15 end.  Unwritten slots keep
// what the workspace held.
constexpr int kWgClockSlots = 16;
#if FD_WG_TIMING
#define FD_MARK(args, slot)                                                                              \
    do {                                                                                                 \
        if (threadIdx.x == 0 && (args).wg_clock && (slot) < kWgClockSlots)                               \
            (args).wg_clock[(size_t)blockIdx.x * kWgClockSlots + (slot)] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
#else
#define FD_MARK(args, slot) \
    do {                    \
    } while (0)
#endif

// Most sequences a stream-mode launch handles (its LDS prefix array).
constexpr int kStreamMaxB = 2048;

struct CombineArgs {
    const float *part_o;
    const float *part_m;
    const float *part_l;
    const int32_t *seq_lens;
    float *out;
    float *lse;
    int B, Hq, T, D;
    int Hkv, G, nq, R;           // partial row p = (b * Hkv + kv head) * R + row
    int n_splits, chunk;
    const int32_t *dev_chunk;    // query-tiled partials: the chunk the order pass chose (nullptr: chunk)
    int append;                  // sequences hold seq_lens[b] + 1 tokens
    int causal;                  // query r / G sees T_b - (nq - 1 - r / G) tokens:
                                 // only splits that start below that are read
    int per_wave;                // 1: half a wave per row (many rows, few splits)
};

// Shape constants of the vector-ALU split kernel.  Each 64-lane wavefront
// reads whole 16-byte pieces of key/value rows: LPR lanes cover one row,
// so a wave holds R rows (tokens) at a time and U tokens per row per step.
template <int EB, int D, int GB>
struct ValuShape {
    static constexpr int ROWB = D * EB;                     // bytes per token row
    static constexpr int LPR = ROWB / 16 < 16 ? ROWB / 16 : 16;
    static constexpr int VEC = ROWB / (16 * LPR);           // 16-B pieces per lane
    static constexpr int EPC = 16 / EB;                     // elements per piece
    static constexpr int EPT = VEC * EPC;                   // elements per lane
    static constexpr int R = 64 / LPR;                      // rows per wave
    static constexpr int U = GB >= 4 ? 2 : FD_VALU_U;       // tokens per row per step
    static constexpr int WAVES = 4;
    static constexpr int TW = R * U;                        // tokens per wave step
    static constexpr int TILE = WAVES * TW;                 // tokens per workgroup step
    static constexpr int THREADS = 64 * WAVES;
};

// Tokens per workgroup step of the VALU kernel instance (host side).
int valu_tile(int dtype, int D, int heads_per_block);
// Launch the VALU split kernel.  Returns the HIP status of the launch.
hipError_t launch_split_valu(const SplitArgs &a, int dtype, hipStream_t stream);

// Matrix-core split kernel (f16 / bf16): up to 16 query heads of one kv head
// per workgroup, 32 tokens per wave step, four waves.
constexpr int kMfmaHeads = 16;
constexpr int kMfmaTile = 128;
hipError_t launch_split_mfma(const SplitArgs &a, int dtype, hipStream_t stream);
// Launch the combine kernel.
hipError_t launch_combine(const CombineArgs &a, hipStream_t stream);

// Many queries per sequence (prefill): one workgroup per tile of
// kPrefillRows query rows of one (batch, kv head) and split of the KV axis,
// over the split's visible tokens in tiles of kPrefillTokens tokens staged
// in LDS.  With one split the workgroup normalises and writes out / lse;
// with several it leaves partials in the combine kernel's layout.
#ifndef FD_PREFILL_NB
#define FD_PREFILL_NB 2
#endif
constexpr int kPrefillNB = FD_PREFILL_NB;          // 16-row blocks per wave
constexpr int kPrefillRows = 64 * kPrefillNB;
// Tile of one 16-row block per wave, for 64 or fewer query rows per kv
// head (value product without converted V only).
constexpr int kPrefillSmallRows = 64;
constexpr int kPrefillTokens = 32;

struct PrefillArgs {
    const void *q;               // [B, nq, Hq, D]
    const void *k;
    const void *v;
    const int32_t *page_table;   // nullptr: contiguous cache
    const int32_t *seq_lens;     // nullptr: every sequence has length T
    float *out;                  // [B, nq, Hq, D]
    float *lse;                  // [B, nq, Hq], may be nullptr
    int B, nq, Hq, Hkv, T, D, G;
    int R;                       // query rows per kv head = nq * G
    int tile_rows;               // query rows per workgroup: kPrefillRows or kPrefillSmallRows
    int row_tiles;               // ceil(R / tile_rows)
    int causal;                  // query i sees the first T_b - (nq - 1 - i) tokens
    // KV splits: split s covers tokens [s * chunk, (s + 1) * chunk), chunk a
    // multiple of kPrefillTokens.  n_splits > 1 writes unnormalised partials
    // (row p = (b * Hkv + kv head) * R + query row, slot p * n_splits + s);
    // a split a row tile sees nothing of is skipped (the combine reads a
    // row's splits only up to its visible length).
    int n_splits, chunk;
    float *part_o;               // [B, Hkv, R, n_splits, D]
    float *part_m;               // [B, Hkv, R, n_splits], log2 units
    float *part_l;               // [B, Hkv, R, n_splits]
    int page_size, page_shift, max_pages, num_pages;
    float scale_log2;
    // bf16 inputs: V converted to f16 under a per-(batch, kv head) power-of-
    // two scale 2^k, transposed in tile order (nullptr: V read as given).
    uint16_t *vt;                // [B, Hkv, vt_tiles, D, kPrefillTokens]
    uint32_t *vmax;              // [B, Hkv, vmax_chunks]: largest |V| (bf16 bits) per chunk
    int32_t *vexp;               // [B, Hkv]: k
    int vt_tiles;                // ceil(T / kPrefillTokens)
    int vmax_chunks;             // ceil(T / kVconvChunk)
    int xcd_map;                 // 1: each XCD walks a contiguous run of work items;
                                 // 2: the same in pairs of ranges, tiles interleaved
    int pool32;                  // paged: each pool is under 4 GiB, so rows are
                                 // addressed with 32-bit byte offsets
    // Longest-first order of the (sequence, split) columns (ragged paged
    // calls with one row tile per kv head and several splits; nullptr: the
    // plain order).  Written by a one-workgroup pass ahead of the kernel:
    // entry c is (b << 16 | split) of the c-th column to run, or ~0u for a
    // column that holds no tokens.
    uint32_t *order;
    // With `order`, the order pass may also choose the chunk from the
    // lengths (nullptr: the plan's `chunk`): it writes it here, and the
    // kernel and the combine read it.  `chunk` is then the smallest it may
    // pick (n_splits columns cover T), and `slots` the workgroups resident at
    // once that it balances over.
    int32_t *dev_chunk;
    int slots;
};
constexpr int kOrderMaxB = 1024;                 // sequences the order pass ranks
constexpr int kVconvChunk = 256;                  // tokens per workgroup of the conversion passes

// Workspace of a query-tiled call with converted V (bf16), 256-byte aligned
// pieces: vexp, vmax, vt.
inline size_t prefill_vt_bytes(int B, int Hkv, int T, int D) {
    auto a256 = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t sl = (size_t)B * Hkv;
    const size_t tiles = ((size_t)T + kPrefillTokens - 1) / kPrefillTokens;
    const size_t chunks = ((size_t)T + kVconvChunk - 1) / kVconvChunk;
    return a256(sl * 4) + a256(sl * chunks * 4) + a256(sl * tiles * D * kPrefillTokens * 2);
}

// The column order of a query-tiled call (after the partials).
inline size_t prefill_order_bytes(int B, int n_splits) {
    return ((size_t)B * n_splits * 4 + 255) / 256 * 256 + 256;   // + the chosen chunk
}

// Partials of a query-tiled call with n_splits > 1 (after the converted V
// pieces, if any): part_o, part_m, part_l, 256-byte aligned.
inline size_t prefill_part_bytes(int B, int Hkv, int R, int D, int n_splits) {
    if (n_splits <= 1) return 0;
    auto a256 = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t parts = (size_t)B * Hkv * R * (size_t)n_splits;
    return a256(parts * D * 4) + 2 * a256(parts * 4);
}

hipError_t launch_prefill(const PrefillArgs &a, int dtype, hipStream_t stream);

// Host side of fd_decode_noalloc (fd_api.cpp).  scratch_plan makes every
// check fd_decode makes, plus no caller workspace and a plan that fits the
// static scratch, without touching the device unless num_cus is 0;
// decode_with_scratch then runs fd_decode with the scratch as workspace.
fd_status_t scratch_plan(const void *q, const void *k_cache, const void *v_cache, const int32_t *page_table,
                         const int32_t *seq_lens, float *out, float *lse, int B, int Hq, int Hkv, int T, int D,
                         float scale, int n_splits, const fd_options_t *opt, size_t scratch_bytes);
fd_status_t decode_with_scratch(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *page_table, const int32_t *seq_lens, float *out, float *lse,
                                int B, int Hq, int Hkv, int T, int D, float scale, int n_splits,
                                const fd_options_t *opt, void *scratch, size_t scratch_bytes);
// Record a failure in fd_last_error and return its status.
fd_status_t hip_error(hipError_t e, const char *what);
fd_status_t error(fd_status_t st, const char *msg);

}  // namespace fdk
