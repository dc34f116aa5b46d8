// Query-tiled attention for many queries per sequence (the prefill phase)
// on the gfx950 matrix cores.
//
// The pages contrast the two phases (dupenodi guide "FlashDecoding and
// split-KV", "Concept" and "The big idea"): prefill attends with a whole
// block of queries and wants tiling over the query axis, decode has one
// query and wants the KV axis split.  This kernel is the query-tiled one:
// a workgroup owns a tile of 64 * NB query rows (128; 64 when a kv head
// has no more) of one (batch, kv head) -- the rows are (query, head of the
// GQA group) pairs, so every row of the tile reads the same K and V -- and
// walks the visible KV range in tiles of
// kPrefillTokens tokens with an online softmax (the same running max / sum
// / unnormalised accumulator as the split pass), then divides once.
// Where row tiles alone leave the device short of work (few queries over a
// long cache, or a ragged batch whose longest sequence would set the time),
// the KV axis is split as in decode: a workgroup then covers one split and
// leaves the unnormalised partial with its max and sum, and the combine
// kernel merges a row's splits (tinyvolt "Kernel visualization: Flash
// Decoding", "Combine kernel").
//
// Per KV tile, staged in LDS by the whole workgroup (three buffers: tile j
// being consumed, tile j+1 being read for its logits, tile j+2 being
// stored; global loads run one more tile ahead):
//  * K rows as they are in memory and V transposed, V^T[d][token], so that
//    the value product can take 8 tokens of one dimension per lane in one
//    16-byte read: within a row the tokens are stored in the order the
//    lanes take them (position 8*((t%16)/4) + 4*(t/16) + t%4 for token t).
//    (Paged 64-row tiles with V read as given store V rows as loaded and
//    take the same operand through transposing LDS reads; see VROWS.)
//    Both row strides are padded by 32 bytes: gfx950 serves a 16-byte LDS
//    read 32 lanes at a time over 128 banks, and rows 8 dwords apart (mod
//    128) keep the 16 rows x 2 chunks of such a read on distinct banks,
//    where a 16-byte pad (4 dwords) measured 2-way conflicts.
// Per wave (two blocks of 16 rows, each K / V fragment read from LDS once
// for both) and tile (two 16-token halves):
//  * logits S^T = K Q^T with v_mfma_f32_16x16x32_{bf16,f16}: tokens on M,
//    query rows on N (the q pieces are the B operand, loaded once), so lane
//    (i16, kb) holds row i16's logits of tokens 4*kb .. 4*kb+3 of each half;
//    the logits of tile j+1 are formed while tile j's softmax runs;
//  * online softmax in base 2 per row: max over the lane's 8 logits, then
//    (only when the running max must move) across the four lanes of the row;
//  * values O^T += V^T P^T with the same MFMA: V^T rows from LDS as the A
//    operand, P^T from the lane's own probabilities as the B operand (k slot
//    8*kb + e is token 4*kb + e of the first half for e < 4, of the second
//    half for e >= 4, on both operands).  P goes in once, rounded to f16
//    (11 significant bits, to nearest).  bf16 V is first converted to f16 by
//    two passes (the end of this file) under a per-(batch, kv head) power of
//    two, exact for every value that matters; without that conversion a bf16
//    P would be needed, and it goes in as a high and a low part (P = hi + lo,
//    two MFMAs) so that its rounding stays near fp32.
//    The accumulator leaves lane (i16, kb) holding row i16's dimensions
//    16*dt + 4*kb .. +3, written out as one 16-byte store per tile of 16.
// Causal rows (query i sees the first T_b - (nq - 1 - i) tokens) are masked
// per element; a workgroup stops at the last token any of its rows sees, and
// the grid runs the longest tiles first.
#include <type_traits>

#include "fd_kernels.h"



namespace fdk {
namespace {

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309417f;

template <int DT>
__device__ __forceinline__ f32x4_v mfma(const uint4 &a, const uint4 &b, f32x4_v c) {
    if constexpr (DT == FD_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a),
                                                       __builtin_bit_cast(bf16x8_v, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_v, a),
                                                      __builtin_bit_cast(f16x8_v, b), c, 0, 0, 0);
}

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));

// Two finite fp32 values as packed 16-bit storage values, rounded to
// nearest (one instruction each way on gfx950).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
    if constexpr (DT == FD_BF16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{x, y}, bf16x2_v));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{x, y}, f16x2_v));
}

// The two bf16 halves of a packed word as fp32 (exact).
__device__ __forceinline__ void unpack2_bf16(uint32_t w, float &x, float &y) {
    x = __uint_as_float(w << 16);
    y = __uint_as_float(w & 0xffff0000u);
}

// max(a, b, c) with NaN propagation: one v_maximum3_f32, no canonicalising
// moves in front of it.
__device__ __forceinline__ float max3(float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// The running max of a row is only raised when a tile's max exceeds it by
// more than this (log2 units): probabilities then stay below 2^kSlack and
// most tiles skip rescaling the accumulator.
constexpr float kSlack = 8.f;

// VT: bf16 inputs whose V was converted by the passes below to f16 under a
// per-(batch, kv head) power-of-two scale, transposed in tile order; the
// value product then runs on f16 with one P product, as for f16 inputs.
// NB: 16-row blocks per wave (the workgroup's tile is 64 * NB query rows).
// P32: paged pools under 4 GiB, whose rows are loaded through buffer
// resources over the pools with 32-bit byte offsets (as contiguous slices
// are) instead of 64-bit addresses.
template <int DT, int D, bool PAGED, bool VT, int NB, bool P32 = false>
__global__ __launch_bounds__(256, (PAGED && NB == 1 && !VT) ? 3 : 2) void prefill(PrefillArgs a) {
    constexpr int ROWB = D * 2;              // bytes per K / V row
    constexpr int KS = D / 32;               // 32-wide k chunks of the logit product
    constexpr int DT16 = D / 16;             // 16-wide dimension tiles of the value product
    constexpr int PIECES = ROWB / 16;        // 16-byte pieces per row
    constexpr int NTOK = kPrefillTokens;     // tokens per KV tile
    // LDS row strides: gfx950 serves a 16-byte read 32 lanes at a time over
    // 128 banks; 16 rows x 2 chunks land on distinct banks when consecutive
    // rows start 8 dwords apart (mod 128).  A 16-byte pad (4 dwords) measured
    // 2-way conflicts.
    // (paged 64-row tiles with V read as given pad K rows by 16 bytes, so
    // that three workgroups fit a compute unit's LDS)
    constexpr int KSTR = ROWB + ((PAGED && NB == 1 && !VT) ? 16 : 32);   // K (bytes)
    constexpr int VSTR = NTOK * 2 + 32;      // V^T (bytes), converted V
    // Paged 64-row tiles with V read as given store V as loaded (token rows,
    // stride ROWB + 32: 8 x an odd number of dwords) and form the value
    // product's A operand by transposing LDS reads, so no thread transposes
    // V on its way in, and three workgroups fit a compute unit (LDS and 168
    // registers).  Measured, paged ragged batch with 16 causal queries: 528
    // -> 496 us; 8 queries 483 -> 470 us.  Contiguous 64-row tiles measured
    // 2-3% slower that way and 128-row f16 tiles 4% slower, so they keep the
    // transposing stores.
    constexpr bool VROWS = PAGED && NB == 1 && !VT;
    constexpr int VROW = ROWB + 32;
    constexpr int ROWS = 64 * NB;            // query rows of the workgroup's tile
    // The value product takes P rounded to f16 (11 significant bits: weights
    // off by at most 2^-11 relative) -- for f16 inputs, and for bf16 inputs
    // whose V was converted (VT).  Otherwise bf16 P, with 8 bits, would spend
    // the whole output tolerance: it goes in as a high and a low part.
    constexpr bool SPLIT_P = DT == FD_BF16 && !VT;
    constexpr int PVT = VT ? FD_F16 : DT;    // operand type of the value product
    static_assert(!VT || DT == FD_BF16, "only bf16 V is converted");
    // f16 probabilities are formed as 2^(x - m + kPBias), in [0, 2^14]: far
    // above the f16 subnormal range for every weight that matters and below
    // its largest finite value.  The bias cancels in the division by the sum.
    constexpr float kPBias = SPLIT_P ? 0.f : 6.f;
    static_assert(NTOK == 32, "the tile maps assume 32 tokens x 4 waves x NB*16 rows");
    static_assert(PIECES * 16 <= 256 && 256 % (PIECES * 16) == 0, "loader threads cover the pieces evenly");

    constexpr int NBUF = 3;                  // tiles j and j+1 in use, j+2 being stored
    __shared__ __align__(16) unsigned char sK[NBUF][NTOK * KSTR];
    __shared__ __align__(16) unsigned char sV[NBUF][VROWS ? NTOK * VROW : D * VSTR];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int i16 = lane & 15;
    const int kb = lane >> 4;

    // Work item of this workgroup: a K/V range -- (batch, kv head, KV split),
    // numbered split-major -- and a row tile.  Workgroups are dealt to the 8
    // XCDs round-robin by linear id.  With xcd_map, XCD x instead runs the
    // ranges x, x + 8, x + 16, ... in turn, all row tiles of one range
    // back to back: the workgroups it runs at once share a K/V range that
    // its own L2 holds, and the ranges of every sequence and split spread
    // evenly over the XCDs (consecutive kv heads of one split land on
    // different XCDs), however ragged the lengths.  Ranges past the last
    // multiple of 8 keep the plain order.  Within a range causal tiles run
    // longest first; causal calls (xcd_map 2) also take an XCD's ranges in
    // pairs with their tiles interleaved (tile t of both ranges, then t - 1),
    // so that the long tiles of the next ranges do not start behind a run of
    // short ones (list scheduling on one XCD's slots: 4 ranges of 32 tiles
    // end at 1.48x the average load one range after another, at the average
    // load in interleaved pairs) while an XCD still holds about two ranges'
    // K/V at a time.
    // With a column order (one row tile per kv head), consecutive
    // workgroups take the kv heads of one (sequence, split) column, columns
    // in the order the order pass wrote: longest first.
    const int lin = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
    int tile_i, split, kvh, b;
    if (a.order) {
        const uint32_t col = a.order[lin / a.Hkv];
        if (col == ~0u) return;                    // a column without tokens
        tile_i = 0;
        kvh = lin % a.Hkv;
        b = (int)(col >> 16);
        split = (int)(col & 0xffffu);
    } else {
        const int n_rng = a.B * a.Hkv * a.n_splits;
        const int mapped = (n_rng / 8) * 8 * a.row_tiles;
        int item = lin;
        if (a.xcd_map && lin < mapped) {
            const int g = lin / 8;
            if (a.xcd_map == 2) {
                const int nr = n_rng / 8;                  // ranges of this XCD
                const int pair = g / (2 * a.row_tiles);
                const int w = g - pair * 2 * a.row_tiles;
                const int gl = min(2, nr - 2 * pair);      // 1 for the last of an odd count
                item = ((lin % 8) + 8 * (2 * pair + w % gl)) * a.row_tiles + w / gl;
            } else {
                item = ((lin % 8) + 8 * (g / a.row_tiles)) * a.row_tiles + g % a.row_tiles;
            }
        }
        tile_i = item % a.row_tiles;
        const int rng = item / a.row_tiles;
        split = rng / (a.B * a.Hkv);
        const int slc0 = rng - split * (a.B * a.Hkv);
        kvh = slc0 % a.Hkv;
        b = slc0 / a.Hkv;
    }
    const int slc = b * a.Hkv + kvh;
    const int tile = a.causal ? a.row_tiles - 1 - tile_i : tile_i;
    const int r0 = tile * ROWS;

    int Tb = a.seq_lens ? a.seq_lens[b] : a.T;
    Tb = Tb < 0 ? 0 : (Tb > a.T ? a.T : Tb);

    // A negative scale is folded into q: flipping the sign of every element
    // is exact, and the exponent's multiplier is then never negative, so a
    // row's largest scaled logit is its largest logit times the multiplier.
    const bool neg = a.scale_log2 < 0.f;
    const float sl2 = neg ? -a.scale_log2 : a.scale_log2;
    const uint32_t qflip = neg ? 0x80008000u : 0u;

    // Output row of a lane's query row in block nb (recomputed after the
    // loop rather than kept live through it).
    auto row_of = [&](int nb, bool &ok) -> size_t {
        const int rr = r0 + 16 * (NB * wave + nb) + i16;
        ok = rr < a.R;
        const int qi = ok ? rr / a.G : 0;
        return ((size_t)b * a.nq + qi) * a.Hq + (size_t)kvh * a.G + (ok ? rr - qi * a.G : 0);
    };
    // This lane's query rows (one per block): the tokens each sees and its
    // q pieces.
    int lim[NB];
    uint4 qb[NB][KS];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        bool ok;
        const size_t qrow = row_of(nb, ok);
        const int qi = ok ? (r0 + 16 * (NB * wave + nb) + i16) / a.G : 0;
        int lm = 0;
        if (ok) lm = a.causal ? Tb - (a.nq - 1 - qi) : Tb;
        lim[nb] = lm < 0 ? 0 : lm;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 w = ok ? *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.q) +
                                                           qrow * ROWB + (4 * ks + kb) * 16)
                                 : make_uint4(0, 0, 0, 0);
            w.x ^= qflip; w.y ^= qflip; w.z ^= qflip; w.w ^= qflip;
            qb[nb][ks] = w;
        }
    }

    // Tokens every row of this wave sees (0 if the wave has rows past R):
    // tiles below it need no mask.
    int wave_lim = 0;
    {
        const int rw0 = r0 + 16 * NB * wave;
        if (rw0 + 16 * NB <= a.R) {
            wave_lim = a.causal ? Tb - (a.nq - 1 - rw0 / a.G) : Tb;
            wave_lim = wave_lim < 0 ? 0 : wave_lim;
        }
    }

    // Tokens the workgroup's rows see at most, and its tiles [j0, j1) of
    // them: the split's.
    const int r_last = min(r0 + ROWS, a.R) - 1;
    int seen = a.causal ? Tb - (a.nq - 1 - r_last / a.G) : Tb;
    seen = seen < 0 ? 0 : seen;
    const bool parts = a.n_splits > 1;
    const int chunk_t = (a.dev_chunk ? *a.dev_chunk : a.chunk) / NTOK;   // tiles per split
    const int j0 = parts ? split * chunk_t : 0;
    int j1 = (seen + NTOK - 1) / NTOK;
    if (parts) {
        j1 = min(j1, j0 + chunk_t);
        if (j1 <= j0) return;    // no row of the tile sees this split: never read
    }
    const int nt = j1 - j0;

    // Loader: thread t moves tokens 2u, 2u+1 of the tile, piece p of each
    // (with D = 64 two threads share a piece and store the same bytes).  V
    // takes u = t % 16, so the 16 lanes of a store write 16 columns of one
    // V^T row; K takes the piece from t % PIECES, so they write one K row.
    const int u = t & 15;
    const int piece = (t >> 4) % PIECES;
    const int ku = (t / PIECES) % 16;
    const int kpiece = t % PIECES;
    // One tile's worth of this thread's loads.
    struct Regs {
        uint4 k0, k1, v0, v1;
        int ok0, ok1;
    };
    // Paged caches: the page ids this thread needs for tile j -- of its V
    // token pair 2u, 2u+1 and its K token pair 2ku, 2ku+1 (with pages of two
    // or more tokens a pair never straddles a page, so one id serves both).
    // Without converted V they are read one step before the tile's K/V
    // loads, which then do not wait on a dependent page-table read (calls
    // with few rows are bound by those reads).  With converted V (many rows,
    // bound by the matrix cores), and in the f16 128-row instance, they are
    // read just before: there the four registers would spill.  Tokens past
    // the end are clamped to the last real one (Tb >= 1 wherever a tile is
    // loaded), so every read is in bounds.
    constexpr bool PREFETCH_PAGES = PAGED && !VT && (NB == 1 || DT == FD_BF16);
    struct Pages {
        int v0, v1, k0, k1;
    };
    auto fetch_pages = [&](int j) -> Pages {
        Pages pp{0, 0, 0, 0};
        if constexpr (PAGED) {
            auto pid = [&](int tt) {
                const int tc = tt < Tb ? tt : Tb - 1;
                return a.page_table[(size_t)b * a.max_pages + (tc >> a.page_shift)];
            };
            const int tv = j * NTOK + 2 * u, tk = j * NTOK + 2 * ku;
            pp.v0 = pid(tv);
            pp.k0 = pid(tk);
            if (a.page_shift == 0) {
                pp.v1 = pid(tv + 1);
                pp.k1 = pid(tk + 1);
            } else {
                pp.v1 = pp.v0;
                pp.k1 = pp.k0;
            }
        }
        return pp;
    };
    // Row of token tt on page pg, clamped as above; ok = false for a token
    // past the end or on a page outside the pool (read from page 0).
    auto page_row = [&](int pg, int tt, int &ok) -> size_t {
        const int tc = tt < Tb ? tt : Tb - 1;
        const bool valid = (unsigned)pg < (unsigned)a.num_pages;
        ok = (tt < Tb) & valid;
        return ((size_t)(valid ? pg : 0) * a.Hkv + kvh) * a.page_size + (tc & (a.page_size - 1));
    };
    // P32: the same row as a 32-bit byte offset into the pool (the host
    // takes this form only when the pool is under 4 GiB).
    [[maybe_unused]] const uint32_t page_rows = (uint32_t)(a.Hkv * a.page_size);
    [[maybe_unused]] const uint32_t head_row = (uint32_t)(kvh * a.page_size);
    auto page_off = [&](int pg, int tt, int &ok) -> uint32_t {
        const int tc = tt < Tb ? tt : Tb - 1;
        const bool valid = (unsigned)pg < (unsigned)a.num_pages;
        ok = (tt < Tb) & valid;
        return ((uint32_t)(valid ? pg : 0) * page_rows + head_row + (uint32_t)(tc & (a.page_size - 1))) *
               (uint32_t)ROWB;
    };
    // Contiguous caches: the (batch, kv head) slices of K and V as buffer
    // resources sized to the real tokens.  Rows past the end read as zeros
    // (and are masked), so no clamp is needed, and each load takes one
    // 32-bit offset: the tile's (uniform) plus the lane's (constant).  Sizes
    // and offsets are unsigned 32-bit (the host keeps each slice below 4
    // GiB); an offset that wraps past 2^32 lands inside the slice or past its
    // end (zeros), never outside the resource.
    const size_t slice = PAGED ? 0 : ((size_t)b * a.Hkv + kvh) * (size_t)a.T * ROWB;
    const uint32_t n_bytes = PAGED ? 0u : (uint32_t)Tb * (uint32_t)ROWB;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(a.k)) + slice, 0, (int)n_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(a.v)) + slice, 0, (int)n_bytes, 0x00020000);
    const uint32_t kofs = (uint32_t)(2 * ku * ROWB + kpiece * 16);
    const uint32_t vofs = (uint32_t)(2 * u * ROWB + piece * 16);
    // Converted V: tile j of the slice is D rows of 32 f16 (64 bytes, tokens
    // in the order the lanes take them); thread t moves 32 bytes of row
    // (t / 2) % D, half t % 2.  Tiles past the sequence read as zeros.
    const int vtrow = (t >> 1) % D, vthalf = t & 1;
    [[maybe_unused]] int vexp = 0;               // V was scaled by 2^vexp
    [[maybe_unused]] __amdgpu_buffer_rsrc_t rvt = rv;
    if constexpr (VT) {
        const size_t sl = (size_t)b * a.Hkv + kvh;
        const uint32_t vt_bytes = (uint32_t)((Tb + NTOK - 1) / NTOK) * (uint32_t)(D * 64);
        rvt = __builtin_amdgcn_make_buffer_rsrc(a.vt + sl * (size_t)a.vt_tiles * D * 32, 0, (int)vt_bytes,
                                                0x00020000);
        vexp = a.vexp[sl];
    }
    [[maybe_unused]] __amdgpu_buffer_rsrc_t rkp = rk, rvp = rv;
    if constexpr (PAGED && P32) {
        const uint32_t pool = (uint32_t)a.num_pages * page_rows * (uint32_t)ROWB;
        rkp = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(static_cast<const char *>(a.k)), 0, (int)pool,
                                                0x00020000);
        rvp = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(static_cast<const char *>(a.v)), 0, (int)pool,
                                                0x00020000);
    }
    auto bload = [](__amdgpu_buffer_rsrc_t r, uint32_t off) -> uint4 {
        typedef unsigned u32x4_v __attribute__((ext_vector_type(4)));
        const u32x4_v x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
        return make_uint4(x[0], x[1], x[2], x[3]);
    };
    auto load_tile = [&](int j, [[maybe_unused]] const Pages &pp) -> Regs {
        Regs g;
        if constexpr (!PAGED) {
            const uint32_t base = (uint32_t)j * (uint32_t)(NTOK * ROWB);
            g.k0 = bload(rk, base + kofs);
            g.k1 = bload(rk, base + kofs + ROWB);
            if constexpr (VT) {
                const uint32_t vb = (uint32_t)j * (uint32_t)(D * 64) + (uint32_t)(vtrow * 64 + vthalf * 32);
                g.v0 = bload(rvt, vb);
                g.v1 = bload(rvt, vb + 16);
            } else {
                g.v0 = bload(rv, base + vofs);
                g.v1 = bload(rv, base + vofs + ROWB);
            }
            g.ok0 = g.ok1 = 1;                   // unused: the row limits mask the tail
            return g;
        }
        int unused_ok;                           // the mask bits come from the V rows
        const int tv = j * NTOK + 2 * u, tk = j * NTOK + 2 * ku;
        if constexpr (P32) {
            [[maybe_unused]] const uint32_t oa = page_off(pp.v0, tv, g.ok0);
            [[maybe_unused]] const uint32_t ob = page_off(pp.v1, tv + 1, g.ok1);
            g.k0 = bload(rkp, page_off(pp.k0, tk, unused_ok) + (uint32_t)(kpiece * 16));
            g.k1 = bload(rkp, page_off(pp.k1, tk + 1, unused_ok) + (uint32_t)(kpiece * 16));
            if constexpr (VT) {
                const uint32_t vb = (uint32_t)j * (uint32_t)(D * 64) + (uint32_t)(vtrow * 64 + vthalf * 32);
                g.v0 = bload(rvt, vb);
                g.v1 = bload(rvt, vb + 16);
            } else {
                g.v0 = bload(rvp, oa + (uint32_t)(piece * 16));
                g.v1 = bload(rvp, ob + (uint32_t)(piece * 16));
            }
            return g;
        }
        [[maybe_unused]] const size_t ra = page_row(pp.v0, tv, g.ok0);
        [[maybe_unused]] const size_t rb = page_row(pp.v1, tv + 1, g.ok1);
        const size_t ka = page_row(pp.k0, tk, unused_ok);
        const size_t kb2 = page_row(pp.k1, tk + 1, unused_ok);
        const char *kp = static_cast<const char *>(a.k) + kpiece * 16;
        [[maybe_unused]] const char *vp = static_cast<const char *>(a.v) + piece * 16;
        g.k0 = *reinterpret_cast<const uint4 *>(kp + ka * ROWB);
        g.k1 = *reinterpret_cast<const uint4 *>(kp + kb2 * ROWB);
        if constexpr (VT) {
            const uint32_t vb = (uint32_t)j * (uint32_t)(D * 64) + (uint32_t)(vtrow * 64 + vthalf * 32);
            g.v0 = bload(rvt, vb);
            g.v1 = bload(rvt, vb + 16);
        } else {
            g.v0 = *reinterpret_cast<const uint4 *>(vp + ra * ROWB);
            g.v1 = *reinterpret_cast<const uint4 *>(vp + rb * ROWB);
        }
        return g;
    };
    // Paged tiles: bit t is set when token t of the tile is real and its
    // page lies in the pool.  Lanes 0..15 of every wave hold tokens 2u, 2u+1
    // of u = lane, so each wave forms the word itself, in scalar registers.
    auto tile_bits = [](const Regs g) -> uint32_t {
        auto spread = [](uint32_t x) {
            x = (x | (x << 8)) & 0x00FF00FFu;
            x = (x | (x << 4)) & 0x0F0F0F0Fu;
            x = (x | (x << 2)) & 0x33333333u;
            return (x | (x << 1)) & 0x55555555u;
        };
        const uint32_t b0 = (uint32_t)__ballot(g.ok0) & 0xffffu;
        const uint32_t b1 = (uint32_t)__ballot(g.ok1) & 0xffffu;
        return spread(b0) | (spread(b1) << 1);
    };
    // V^T column of token tt of a tile (see the header): tokens 2u and 2u+1
    // stay adjacent, so one 32-bit store writes both.
    auto vpos = [](int tt) { return 8 * ((tt & 15) >> 2) + 4 * (tt >> 4) + (tt & 3); };
    auto store_tile = [&](int buf, const Regs g) {
        *reinterpret_cast<uint4 *>(&sK[buf][(2 * ku) * KSTR + kpiece * 16]) = g.k0;
        *reinterpret_cast<uint4 *>(&sK[buf][(2 * ku + 1) * KSTR + kpiece * 16]) = g.k1;
        if constexpr (VT) {
            // already transposed and in lane order: a plain copy
            *reinterpret_cast<uint4 *>(&sV[buf][vtrow * VSTR + vthalf * 32]) = g.v0;
            *reinterpret_cast<uint4 *>(&sV[buf][vtrow * VSTR + vthalf * 32 + 16]) = g.v1;
            return;
        }
        if constexpr (VROWS) {
            // token rows 2u, 2u+1, piece `piece`, as loaded
            *reinterpret_cast<uint4 *>(&sV[buf][(2 * u) * VROW + piece * 16]) = g.v0;
            *reinterpret_cast<uint4 *>(&sV[buf][(2 * u + 1) * VROW + piece * 16]) = g.v1;
            return;
        }
        // V^T: dimension 8*piece + e, tokens 2u and 2u+1 packed in one word
        const uint32_t w0[4] = {g.v0.x, g.v0.y, g.v0.z, g.v0.w};
        const uint32_t w1[4] = {g.v1.x, g.v1.y, g.v1.z, g.v1.w};
        const int col = 2 * vpos(2 * u);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<uint32_t *>(&sV[buf][(8 * piece + 2 * i) * VSTR + col]) =
                (w0[i] & 0xffffu) | (w1[i] << 16);
            *reinterpret_cast<uint32_t *>(&sV[buf][(8 * piece + 2 * i + 1) * VSTR + col]) =
                (w0[i] >> 16) | (w1[i] & 0xffff0000u);
        }
    };

    // Per row: the running max m (log2 units), m + kSlack, the exponent
    // offset kPBias - m (kPBias while m = -inf), the sum and the accumulator.
    f32x4_v acc[NB][DT16];
    float m[NB], mth[NB], nm[NB], l[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int dt = 0; dt < DT16; ++dt) acc[nb][dt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
        m[nb] = mth[nb] = kNegInf;
        nm[nb] = kPBias;
        l[nb] = 0.f;
    }

    // Logits of the tile in LDS buffer `buf` for all row blocks; each K
    // fragment is read once.
    auto qk = [&](int buf, f32x4_v (&c)[NB][2]) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) c[nb][0] = c[nb][1] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint4 kp = *reinterpret_cast<const uint4 *>(&sK[buf][(16 * h + i16) * KSTR + (4 * ks + kb) * 16]);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) c[nb][h] = mfma<DT>(kp, qb[nb][ks], c[nb][h]);
            }
    };

    Regs g{};
    uint32_t ok_cur = 0, ok_next = 0;       // paged mask words of tiles j, j+1
    Pages pnext{0, 0, 0, 0};                // paged, prefetching: page ids of the next tile to load

    // One tile: step j consumes the logits cc of tile j (formed one step
    // earlier) and forms cn, those of tile j+1.
    //  1. masks, row maxima and (rarely) the rescale -- the only branches;
    //  2. one straight-line block: tile j+2 (loaded one step earlier) into
    //     its LDS buffer, tile j+3 from memory, logits of tile j+1, and the
    //     probabilities and value product of tile j.  Past the last tile the
    //     loads read clamped rows (or zeros) and the logits go unused, so nothing there
    //     needs a branch, and the matrix-core work of the logits can be
    //     interleaved with the vector work of the probabilities.
    // End of a tile step: tile j+2 (loaded one step earlier) into its LDS
    // buffer, whose previous tile j-1 is finished; tile j+3 from memory.
    auto stage_next = [&](auto bjc, const int j) {
        constexpr int bj = decltype(bjc)::value;
        store_tile((bj + 2) % NBUF, g);
        if constexpr (PREFETCH_PAGES) {
            g = load_tile(j + 3, pnext);
            pnext = fetch_pages(j + 4);
        } else {
            g = load_tile(j + 3, fetch_pages(j + 3));
        }
        __syncthreads();
    };
    auto step = [&](auto bjc, const int j, const f32x4_v (&cc)[NB][2], f32x4_v (&cn)[NB][2]) {
        constexpr int bj = decltype(bjc)::value;   // j % NBUF, known at compile time
        // Masks: tiles every row of the wave sees in full need none; there
        // the raw logits are kept and the scale goes into the exponent
        // (p = 2^(x * mult + nm)).  Masked tiles hold scaled logits with -inf
        // for masked tokens (mult = 1).
        // (paged tiles also need every page in the pool)
        const bool full = (j + 1) * NTOK <= wave_lim && (!PAGED || ok_cur == 0xffffffffu);
        const float mult = full ? sl2 : 1.f;
        float x[NB][8];
        if (full) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int e = 0; e < 8; ++e) x[nb][e] = cc[nb][e >> 2][e & 3];
        } else {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int rel = lim[nb] - j * NTOK;    // this row sees tokens [0, rel) of the tile
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int tk = 16 * (e >> 2) + 4 * kb + (e & 3);
                    bool ok = tk < rel;
                    if constexpr (PAGED) ok = ok & (((ok_cur >> tk) & 1u) != 0u);
                    x[nb][e] = ok ? cc[nb][e >> 2][e & 3] * sl2 : kNegInf;
                }
            }
        }
        // The running max of a row moves only when one of its logits exceeds
        // it by more than kSlack; then (rarely, after the first tiles) the
        // row max is formed across its four lanes and the state rescaled.
        float lmt[NB];
        bool need = false;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            lmt[nb] = __builtin_elementwise_maximum(max3(x[nb][0], x[nb][1], x[nb][2]),
                                                    max3(max3(x[nb][3], x[nb][4], x[nb][5]), x[nb][6], x[nb][7])) *
                      mult;
            need = need | (lmt[nb] > mth[nb]);
        }
        if (__any(need)) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float mt = lmt[nb];
                mt = fmaxf(mt, __shfl_xor(mt, 16));
                mt = fmaxf(mt, __shfl_xor(mt, 32));
                const bool grow = mt > mth[nb];
                const float m_new = grow ? mt : m[nb];
                const float alpha = grow ? __builtin_amdgcn_exp2f(m[nb] - m_new) : 1.f;   // 0 when m was -inf
                l[nb] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT16; ++dt) acc[nb][dt] *= alpha;
                m[nb] = m_new;
                mth[nb] = m_new + kSlack;
                nm[nb] = m_new == kNegInf ? kPBias : kPBias - m_new;
            }
        }

        // ---- straight-line block ----
        if constexpr (PAGED) {
            const uint32_t ok_new = tile_bits(g);
            ok_cur = ok_next;
            ok_next = ok_new;
        }
        qk((bj + 1) % NBUF, cn);
        uint4 phi[NB], plo[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(x[nb][e], mult, nm[nb]));
            l[nb] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hi[e] = pack2<PVT>(p[2 * e], p[2 * e + 1]);
                if constexpr (SPLIT_P) {
                    float h0, h1;
                    unpack2_bf16(hi[e], h0, h1);
                    lo[e] = pack2<DT>(p[2 * e] - h0, p[2 * e + 1] - h1);   // exact differences
                }
            }
            // P^T as the B operand (in two 16-bit parts for bf16)
            phi[nb] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            if constexpr (SPLIT_P) plo[nb] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
        // Paged 64-row tiles with V read as given: a wave raises its issue
        // priority for its value product (back to 0 before the staging), so
        // among the 12 waves of a compute unit the one holding P issues its
        // MFMAs first (measured, paged ragged batch with 16 causal queries:
        // 457 -> 445 us; 8 queries 433 -> 425).  The f16 form measured no
        // faster and the 128-row tiles slower (GQA, 4096 queries: 1164 ->
        // 1184 us), so they keep one priority.
        if constexpr (VROWS && DT == FD_BF16) __builtin_amdgcn_s_setprio(1);
        // values: dimension tiles in pairs (the high parts of P, then the
        // low parts), so consecutive MFMAs never wait on each other; the
        // staging of tile j+2 and the loads of tile j+3 fill the gaps
#pragma unroll
        for (int dt = 0; dt < DT16; dt += 2) {
            uint4 va[2];
#pragma unroll
            for (int y = 0; y < 2; ++y) {
                if constexpr (VROWS) {
                    // ds_read_b64_tr_b16: within each group of 16 lanes, lane
                    // j names 4 consecutive 16-bit values M[j][0..3]; lane i
                    // receives M[4k + i/4][i%4] for k = 0..3 (checked on gfx950
                    // with an index-filled LDS array).  Lane j of group kb names
                    // token 16h + 4kb + j/4, dims 16*(dt+y) + 4*(j%4): lane i16
                    // gets dim 16*(dt+y) + i16 of tokens 4kb .. 4kb+3 (h = 0)
                    // and 16+4kb .. (h = 1), the k slots of the P operand.
                    const unsigned char *rd =
                        &sV[bj][(4 * kb + (i16 >> 2)) * VROW + 32 * (dt + y) + 8 * (i16 & 3)];
                    typedef short i16x4_v __attribute__((ext_vector_type(4)));
                    const uint2 a0 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4_v *)(rd)));
                    const uint2 a1 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4_v *)(rd + 16 * VROW)));
                    va[y] = make_uint4(a0.x, a0.y, a1.x, a1.y);
                } else {
                    va[y] = *reinterpret_cast<const uint4 *>(&sV[bj][(16 * (dt + y) + i16) * VSTR + 16 * kb]);
                }
            }
#pragma unroll
            for (int y = 0; y < 2; ++y)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) acc[nb][dt + y] = mfma<PVT>(va[y], phi[nb], acc[nb][dt + y]);
            if constexpr (SPLIT_P) {
#pragma unroll
                for (int y = 0; y < 2; ++y)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) acc[nb][dt + y] = mfma<DT>(va[y], plo[nb], acc[nb][dt + y]);
            }
        }
        if constexpr (VROWS && DT == FD_BF16) __builtin_amdgcn_s_setprio(0);
        stage_next(bjc, j);
    };

    // The loop runs three tiles per trip, so every LDS buffer index is a
    // compile-time constant (addresses become instruction offsets); the
    // logits rotate through three register sets, two live at a time.
    f32x4_v cA[NB][2], cB[NB][2], cC[NB][2];
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using B2 = std::integral_constant<int, 2>;
    // Tiles are numbered from the sequence start (masks and loads use that
    // index); LDS buffers count from the split's first tile.
    if (nt > 0) {
        if constexpr (PAGED) {
            const Pages p0 = fetch_pages(j0), p1 = fetch_pages(j0 + 1), p2 = fetch_pages(j0 + 2);
            if constexpr (PREFETCH_PAGES) pnext = fetch_pages(j0 + 3);
            Regs g0 = load_tile(j0, p0);
            ok_cur = tile_bits(g0);
            store_tile(0, g0);
            Regs g1 = load_tile(j0 + 1, p1);
            ok_next = tile_bits(g1);
            store_tile(1, g1);
            g = load_tile(j0 + 2, p2);
        } else {
            store_tile(0, load_tile(j0, pnext));
            store_tile(1, load_tile(j0 + 1, pnext));
            g = load_tile(j0 + 2, pnext);
        }
        __syncthreads();
        int j = 0;
        if (NB == 1 && r0 + 16 * NB * wave >= a.R) {
            // every row block of this wave is past the last row: it computes
            // nothing and only helps stage the tiles, through the same
            // barriers (the wave index is uniform, so is the branch).  Only
            // the 64-row tiles of few-row calls take this form (in 128-row
            // tiles it would make the paged instance spill, and a tile there
            // idles waves only when it is a kv head's last)
            for (; j + 3 <= nt; j += 3) {
                stage_next(B0{}, j0 + j);
                stage_next(B1{}, j0 + j + 1);
                stage_next(B2{}, j0 + j + 2);
            }
            if (j < nt) stage_next(B0{}, j0 + j);
            if (j + 1 < nt) stage_next(B1{}, j0 + j + 1);
        } else {
            qk(0, cA);
            for (; j + 3 <= nt; j += 3) {
                step(B0{}, j0 + j, cA, cB);
                step(B1{}, j0 + j + 1, cB, cC);
                step(B2{}, j0 + j + 2, cC, cA);
            }
            if (j < nt) step(B0{}, j0 + j, cA, cB);
            if (j + 1 < nt) step(B1{}, j0 + j + 1, cB, cC);
        }
    }

    // The four lanes of a row share m; their sums cover different tokens.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        float L = l[nb];
        L += __shfl_xor(L, 16);
        L += __shfl_xor(L, 32);
        bool ok;
        const size_t qrow = row_of(nb, ok);
        if (!ok) continue;
        if (parts) {
            // unnormalised partial of this split, in the units of V; with the
            // bias moved into the max, l = sum 2^(s - m) and o = sum 2^(s - m) v
            const size_t pr = ((size_t)slc * a.R + (r0 + 16 * (NB * wave + nb) + i16)) * a.n_splits + split;
#pragma unroll
            for (int dt = 0; dt < DT16; ++dt) {
                f32x4_v o = acc[nb][dt];
                if constexpr (VT) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = __builtin_amdgcn_ldexpf(o[e], -vexp);
                }
                *reinterpret_cast<float4 *>(a.part_o + pr * D + 16 * dt + 4 * kb) = make_float4(o[0], o[1], o[2], o[3]);
            }
            if (kb == 0) {
                a.part_m[pr] = m[nb] == kNegInf ? kNegInf : m[nb] - kPBias;
                a.part_l[pr] = L;
            }
            continue;
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
        for (int dt = 0; dt < DT16; ++dt) {
            f32x4_v o = acc[nb][dt] * inv;
            if constexpr (VT) {
                // undo the conversion scale exactly (one rounding, also for
                // results in the fp32 subnormal range)
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = __builtin_amdgcn_ldexpf(o[e], -vexp);
            }
            *reinterpret_cast<float4 *>(a.out + qrow * D + 16 * dt + 4 * kb) = make_float4(o[0], o[1], o[2], o[3]);
        }
        if (kb == 0 && a.lse) a.lse[qrow] = L > 0.f ? (m[nb] + log2f(L) - kPBias) * kLn2 : kNegInf;
    }
}

// ---- the longest-first column order ----
// One workgroup of kOrderMaxB threads, thread b for sequence b (B <=
// kOrderMaxB): of the columns (b, s), s < n_splits, those holding a whole
// chunk come first (sequence by sequence; they are all the same work), then
// each sequence's last, partial column by descending token count (ties by
// sequence), then the empty ones (~0u).  The sizes are the cached lengths;
// a causal row tile sees at most that many tokens.
__global__ __launch_bounds__(kOrderMaxB) void order_pass(PrefillArgs a) {
    const int t = threadIdx.x;
    __shared__ int s_rem[kOrderMaxB];
    __shared__ int s_scan[kOrderMaxB];
    __shared__ long long s_sum[kOrderMaxB];
    int Tb = 0;
    if (t < a.B) {
        Tb = a.seq_lens ? a.seq_lens[t] : a.T;
        Tb = Tb < 0 ? 0 : (Tb > a.T ? a.T : Tb);
    }
    int chunk = a.chunk;
    if (a.dev_chunk) {
        // The chunk from the lengths: W tiles of work (every kv head of every
        // sequence), `slots` workgroups at once.  Whole chunks of P tiles with
        // W ~ m * slots * P for a whole number m of rounds pack the slots
        // evenly under longest-first dispatch (the remainders fill in);
        // P is at least the plan's chunk, so n_splits columns still cover
        // every sequence.
        s_sum[t] = t < a.B ? (long long)((Tb + kPrefillTokens - 1) / kPrefillTokens) * a.Hkv : 0;
        __syncthreads();
        for (int off = kOrderMaxB / 2; off > 0; off >>= 1) {
            if (t < off) s_sum[t] += s_sum[t + off];
            __syncthreads();
        }
        const long long W = s_sum[0];
        const long long pmin = a.chunk / kPrefillTokens;
        const long long S = a.slots > 0 ? a.slots : 1;
        long long m = W / (pmin * S);
        if (m < 1) m = 1;
        long long P = (W + m * S - 1) / (m * S);
        if (P < pmin) P = pmin;
        chunk = (int)(P * kPrefillTokens);
        if (t == 0) *a.dev_chunk = chunk;
    }
    const long long cap = (long long)a.n_splits * chunk;
    const int full = t < a.B ? (int)((Tb < cap ? Tb : cap) / chunk) : 0;
    const int rem = (t < a.B && full < a.n_splits) ? Tb - full * chunk : 0;
    s_rem[t] = rem;
    s_scan[t] = full;
    __syncthreads();
    // inclusive scan of the full-column counts
    for (int off = 1; off < kOrderMaxB; off <<= 1) {
        const int x = t >= off ? s_scan[t - off] : 0;
        __syncthreads();
        s_scan[t] += x;
        __syncthreads();
    }
    const int nfull = s_scan[kOrderMaxB - 1];
    const int first = s_scan[t] - full;
    for (int s = 0; s < full; ++s) a.order[first + s] = ((uint32_t)t << 16) | (uint32_t)s;
    if (rem > 0) {
        int rank = 0;
        for (int o = 0; o < a.B; ++o) {
            const int r = s_rem[o];
            rank += (r > rem) | ((r == rem) & (o < t));
        }
        a.order[nfull + rank] = ((uint32_t)t << 16) | (uint32_t)full;
    }
    int npart = 0;
    for (int o = 0; o < a.B; ++o) npart += s_rem[o] > 0;
    for (int c = nfull + npart + t; c < a.B * a.n_splits; c += kOrderMaxB) a.order[c] = ~0u;
}

// ---- bf16 V converted for the value product ----
// A bf16 value v becomes the f16 value v * 2^k, with k chosen per (batch,
// kv head) so that the sequence's largest |v| lands in [2^14, 2^15).  bf16
// keeps 8 significant bits and f16 11, so every value down to 2^-28 of that
// maximum converts exactly (f16 normal range); smaller ones, rounded to the
// f16 subnormal grid, are off by at most 2^-39 of the maximum.  Rounding is
// to nearest; infinities and NaNs stay what they are.

// Pass 1: the largest |V| (bf16 bits, sign cleared) of each chunk of
// kVconvChunk tokens of each (batch, kv head) slice.
template <int D, bool PAGED>
__global__ __launch_bounds__(256) void vmax_pass(PrefillArgs a) {
    constexpr int ROWB = D * 2, PIECES = ROWB / 16, RPI = 256 / PIECES;   // rows per sweep
    const int t = threadIdx.x, chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    int Tb = a.seq_lens ? a.seq_lens[b] : a.T;
    Tb = Tb < 0 ? 0 : (Tb > a.T ? a.T : Tb);
    const int t0 = chunk * kVconvChunk, t1 = min(t0 + kVconvChunk, Tb);
    const int piece = t % PIECES;
    uint32_t mx = 0;
#pragma unroll 4
    for (int tt = t0 + t / PIECES; tt < t1; tt += RPI) {
        size_t row;
        bool ok = true;
        if constexpr (PAGED) {
            const int pg = a.page_table[(size_t)b * a.max_pages + (tt >> a.page_shift)];
            ok = (unsigned)pg < (unsigned)a.num_pages;
            row = ((size_t)(ok ? pg : 0) * a.Hkv + kvh) * a.page_size + (tt & (a.page_size - 1));
        } else {
            row = ((size_t)b * a.Hkv + kvh) * a.T + tt;
        }
        const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.v) + row * ROWB + piece * 16);
        const uint32_t m4 = max(max(w.x & 0x7fff7fffu, w.y & 0x7fff7fffu), max(w.z & 0x7fff7fffu, w.w & 0x7fff7fffu));
        const uint32_t m2 = ok ? max(m4 & 0xffffu, m4 >> 16) : 0u;
        mx = max(mx, m2);
    }
    __shared__ uint32_t red[4];
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
    if ((t & 63) == 0) red[t >> 6] = mx;
    __syncthreads();
    if (t == 0)
        a.vmax[((size_t)b * a.Hkv + kvh) * a.vmax_chunks + chunk] = max(max(red[0], red[1]), max(red[2], red[3]));
}

// Pass 2: the slice's scale exponent k from the chunk maxima, and the
// chunk's tiles converted: tile j is D rows of kPrefillTokens f16, tokens
// in the order the query-tiled kernel's lanes take them; tokens past the
// sequence (or on pages outside the pool) are zeros.
template <int D, bool PAGED>
__global__ __launch_bounds__(256) void vconv_pass(PrefillArgs a) {
    constexpr int ROWB = D * 2, PIECES = ROWB / 16, NTOK = kPrefillTokens;
    const int t = threadIdx.x, chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const size_t sl = (size_t)b * a.Hkv + kvh;
    int Tb = a.seq_lens ? a.seq_lens[b] : a.T;
    Tb = Tb < 0 ? 0 : (Tb > a.T ? a.T : Tb);

    uint32_t mx = 0;
    for (int c = t; c < a.vmax_chunks; c += 256) mx = max(mx, a.vmax[sl * a.vmax_chunks + c]);
    __shared__ uint32_t red[4];
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
    if ((t & 63) == 0) red[t >> 6] = mx;
    __syncthreads();
    mx = max(max(red[0], red[1]), max(red[2], red[3]));
    // floor(log2 of the largest |v|): from the exponent field, or for a
    // subnormal from the top mantissa bit (value = mantissa * 2^-133)
    const int E = (int)(mx >> 7);
    const int lg = E > 0 ? E - 127 : -133 + (31 - __builtin_clz(mx | 1u));
    const int k = mx == 0 ? 0 : 14 - lg;
    if (chunk == 0 && t == 0) a.vexp[sl] = k;

    const int u = t & 15, piece = (t >> 4) % PIECES;   // D = 64: two threads per piece, same values
    const int pos = 8 * ((2 * u & 15) >> 2) + 4 * (2 * u >> 4) + (2 * u & 3);   // lane order of token 2u
    const int nt = (Tb + NTOK - 1) / NTOK;
    const int j0 = chunk * (kVconvChunk / NTOK);
    const int j1 = min(j0 + kVconvChunk / NTOK, nt);
    auto load = [&](int tt) -> uint4 {
        if (tt >= Tb) return make_uint4(0, 0, 0, 0);
        size_t row;
        if constexpr (PAGED) {
            const int pg = a.page_table[(size_t)b * a.max_pages + (tt >> a.page_shift)];
            if ((unsigned)pg >= (unsigned)a.num_pages) return make_uint4(0, 0, 0, 0);
            row = ((size_t)pg * a.Hkv + kvh) * a.page_size + (tt & (a.page_size - 1));
        } else {
            row = ((size_t)b * a.Hkv + kvh) * a.T + tt;
        }
        return *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.v) + row * ROWB + piece * 16);
    };
    auto cvt = [k](float x, float y) -> uint32_t {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                                f32x2_v{__builtin_amdgcn_ldexpf(x, k), __builtin_amdgcn_ldexpf(y, k)},
                                                f16x2_v));
    };
    for (int j = j0; j < j1; ++j) {
        const uint4 v0 = load(j * NTOK + 2 * u), v1 = load(j * NTOK + 2 * u + 1);
        const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w};
        const uint32_t w1[4] = {v1.x, v1.y, v1.z, v1.w};
        uint32_t *tile = reinterpret_cast<uint32_t *>(a.vt + (sl * a.vt_tiles + j) * (size_t)D * NTOK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = 8 * piece + 2 * i;
            tile[(size_t)d * (NTOK / 2) + pos / 2] =
                cvt(__uint_as_float(w0[i] << 16), __uint_as_float(w1[i] << 16));
            tile[(size_t)(d + 1) * (NTOK / 2) + pos / 2] =
                cvt(__uint_as_float(w0[i] & 0xffff0000u), __uint_as_float(w1[i] & 0xffff0000u));
        }
    }
}

template <int DT, int D>
hipError_t launch_dim(const PrefillArgs &a, hipStream_t stream) {
    const dim3 grid(a.row_tiles * a.n_splits, a.Hkv, a.B);
    if (a.order) {
        if (a.row_tiles != 1 || a.B > kOrderMaxB || a.n_splits >= 65536) return hipErrorInvalidValue;
        hipLaunchKernelGGL(order_pass, dim3(1), dim3(kOrderMaxB), 0, stream, a);
    }
    if constexpr (DT == FD_BF16) {
        if (a.vt) {
            if (a.tile_rows != kPrefillRows) return hipErrorInvalidValue;
            const dim3 pgrid(a.vmax_chunks, a.Hkv, a.B);
            if (a.page_table) {
                hipLaunchKernelGGL((vmax_pass<D, true>), pgrid, dim3(256), 0, stream, a);
                hipLaunchKernelGGL((vconv_pass<D, true>), pgrid, dim3(256), 0, stream, a);
            } else {
                hipLaunchKernelGGL((vmax_pass<D, false>), pgrid, dim3(256), 0, stream, a);
                hipLaunchKernelGGL((vconv_pass<D, false>), pgrid, dim3(256), 0, stream, a);
            }
            if (a.page_table && a.pool32)
                hipLaunchKernelGGL((prefill<DT, D, true, true, kPrefillNB, true>), grid, dim3(256), 0, stream, a);
            else if (a.page_table)
                hipLaunchKernelGGL((prefill<DT, D, true, true, kPrefillNB>), grid, dim3(256), 0, stream, a);
            else hipLaunchKernelGGL((prefill<DT, D, false, true, kPrefillNB>), grid, dim3(256), 0, stream, a);
            return hipGetLastError();
        }
    }
    if (a.tile_rows == 64 * kPrefillNB) {
        if (a.page_table && a.pool32)
            hipLaunchKernelGGL((prefill<DT, D, true, false, kPrefillNB, true>), grid, dim3(256), 0, stream, a);
        else if (a.page_table)
            hipLaunchKernelGGL((prefill<DT, D, true, false, kPrefillNB>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((prefill<DT, D, false, false, kPrefillNB>), grid, dim3(256), 0, stream, a);
    } else if (a.tile_rows == kPrefillSmallRows) {
        // a 64-row tile for 33..64 query rows per kv head: no row block idles
        if (a.page_table && a.pool32)
            hipLaunchKernelGGL((prefill<DT, D, true, false, 1, true>), grid, dim3(256), 0, stream, a);
        else if (a.page_table) hipLaunchKernelGGL((prefill<DT, D, true, false, 1>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((prefill<DT, D, false, false, 1>), grid, dim3(256), 0, stream, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dtype(const PrefillArgs &a, hipStream_t stream) {
    switch (a.D) {
    case 64: return launch_dim<DT, 64>(a, stream);
    case 128: return launch_dim<DT, 128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, int dtype, hipStream_t stream) {
    switch (dtype) {
    case FD_F16: return launch_dtype<FD_F16>(a, stream);
    case FD_BF16: return launch_dtype<FD_BF16>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace fdk
