// Split pass of flash decoding on the gfx950 matrix cores, for GQA groups.
//
// Same contract as the VALU split kernel (tinyvolt "Kernel visualization:
// Flash Decoding", single-block walkthrough): one workgroup per (batch, kv
// head, head block, split) streams its chunk of K and V once and leaves an
// unnormalised partial with its running max and sum.  With a GQA group of G
// query heads per kv head, the logits of a 16-token tile are a real
// (16 tokens x D) . (D x G) contraction and the value update a (D x tokens)
// . (tokens x G) one, so both run on MFMA; G is padded to 16.
//
// Per 64-lane wave and 32-token step (two 16-token tiles):
//  * logits: v_mfma_f32_16x16x32_{bf16,f16} with the tile's tokens as the M
//    rows (lane i16 = lane % 16 loads token i16's 16-byte pieces) and the
//    query heads as the N columns (the B operand is the q pieces, loaded
//    once).  Products of two 16-bit values are exact in fp32.  The output
//    leaves lane (i16, kb = lane / 16) holding head i16's logits of tokens
//    4*kb .. 4*kb+3 of the tile, so each lane owns one head;
//  * online softmax: per-lane max over its 8 logits, then across the four
//    lanes of the head (xor 16, xor 32); every lane keeps its own partial
//    sum (all four share the max), summed once at the end;
//  * values: v_mfma_f32_16x16x4f32 in fp32 with P straight from the logit
//    registers as the B operand (no rounding of P, no data movement): for
//    the token group of row r, lane (i16, kb) supplies p of its head and
//    token 4*kb+r, and V of that token as the A operand -- 8 (D=128) or 4
//    (D=64) consecutive elements of the row, one per MFMA, so element i of
//    lane i16 is dimension (D/16)*i16 + i.  Each V load instruction reads
//    four whole rows.  With two row blocks (17-32 rows) the value product
//    instead runs on v_mfma_f32_16x16x32_{bf16,f16}: V^T from LDS through
//    transposing reads as the A operand, P in a high and a low 16-bit part
//    as the B operand (see TRV below);
// The next step's K/V pieces are prefetched into registers while the current
// step is consumed (two buffers used in turn).
#include <type_traits>

#include "fd_epilogue.h"

namespace fdk {
namespace {

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();

template <int DT>
__device__ __forceinline__ f32x4_v mfma_logits(const uint4 &k, const uint4 &q, f32x4_v c) {
    if constexpr (DT == FD_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, k),
                                                       __builtin_bit_cast(bf16x8_v, q), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_v, k),
                                                      __builtin_bit_cast(f16x8_v, q), c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ float widen1(uint32_t w, int hi) {
    if constexpr (DT == FD_BF16) {
        return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16));
    } else {
        return (float)__builtin_bit_cast(_Float16, (unsigned short)(hi ? (w >> 16) : (w & 0xffffu)));
    }
}

template <int DT>
__device__ __forceinline__ void widen(const uint4 &p, float *f) {
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = widen1<DT>(w[i], 0); f[2 * i + 1] = widen1<DT>(w[i], 1); }
}

template <int DT>
__device__ __forceinline__ void widen(const uint2 &p, float *f) {
    const uint32_t w[2] = {p.x, p.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) { f[2 * i] = widen1<DT>(w[i], 0); f[2 * i + 1] = widen1<DT>(w[i], 1); }
}

typedef unsigned int u32x4_v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_v __attribute__((ext_vector_type(2)));
typedef short i16x4_v __attribute__((ext_vector_type(4)));

// Two probabilities as one word of the input type (round to nearest), and
// that word's two values back in fp32 (exact).
template <int DT>
__device__ __forceinline__ uint32_t pack_p(float x, float y) {
    if constexpr (DT == FD_BF16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{x, y}, bf16x2_v));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{x, y}, f16x2_v));
}

template <int DT>
__device__ __forceinline__ void unpack_p(uint32_t w, float &x, float &y) {
    x = widen1<DT>(w, 0);
    y = widen1<DT>(w, 1);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j names 4
// consecutive 16-bit values M[j][0..3]; lane i receives M[4k + i/4][i%4]
// for k = 0..3 (checked on gfx950 with an index-filled LDS array).
__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char *p) {
    const i16x4_v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_v *)(p));
    return __builtin_bit_cast(uint2, v);
}

template <typename V>
__device__ __forceinline__ V load_piece(const char *p);

template <>
__device__ __forceinline__ uint4 load_piece<uint4>(const char *p) {
#if FD_NT_LOADS
    const u32x4_v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_v *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
#else
    return *reinterpret_cast<const uint4 *>(p);
#endif
}

template <>
__device__ __forceinline__ uint2 load_piece<uint2>(const char *p) {
#if FD_NT_LOADS
    const u32x2_v v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_v *>(p));
    return make_uint2(v.x, v.y);
#else
    return *reinterpret_cast<const uint2 *>(p);
#endif
}

// PG: 0 contiguous cache, 1 paged with per-token page lookups (pages under
// 16 tokens), 2 paged with one lookup per 16-token block (pages of 16+).
// STREAM: balanced stream mode (ragged batches), else one workgroup per
// (batch, kv head, head block, split).
// NB: 16-row blocks of query rows per workgroup (1 or 2).  Both blocks use
// the same K and V operands, so 32 query rows still read the KV once; the
// second block's accumulators need the register file of one workgroup per
// compute unit.
template <int DT, int D, int PG, bool STREAM, int NB>
__global__ __launch_bounds__(256, NB == 1 ? 2 : 1) void split_mfma(SplitArgs a) {
    constexpr bool PAGED = PG != 0;
    constexpr int EB = 2;
    constexpr int ROWB = D * EB;
    constexpr int KS = D / 32;          // 16-byte q/k pieces per lane per tile
    constexpr int PVE = D / 16;         // V elements per lane per token
    constexpr int VB = PVE * EB;        // V bytes per lane per token
    constexpr int WAVES = 4;
    constexpr int TOK = 32;             // tokens per wave step
    constexpr int TILE = WAVES * TOK;
    constexpr int GB = kMfmaHeads * NB;
    static_assert(TILE == kMfmaTile, "host and kernel disagree on the tile");
    using VP = typename std::conditional<VB == 16, uint4, uint2>::type;
    using Off = typename std::conditional<PAGED, size_t, uint32_t>::type;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
    const int i16 = lane & 15;
    const int kb = lane >> 4;

    __shared__ int s_pages[PAGED ? kMaxSplitPages : 1];
    __shared__ EpilogueLds<WAVES, GB, D> sm;
    // Two row blocks: the value product runs on 16x16x32 MFMAs, whose A
    // operand needs 8 tokens of one dimension per lane.  Each wave writes its
    // step's V rows (as loaded) to its own LDS tile and reads them back with
    // transposing reads.  Row stride 2D + 32 bytes: 8 x an odd number of
    // dwords, so the 16 token rows one transposing read touches fall on
    // disjoint 8-bank windows of the 128 banks.
    constexpr bool TRV = NB >= 2;
    constexpr int VROW = 2 * D + 32;
    __shared__ __align__(16) unsigned char s_v[TRV ? WAVES : 1][TRV ? TOK * VROW : 16];

    // One segment: tokens [c0, c1) of row (b, kvh, hb) into `so`.
    auto segment = [&](int b, int kvh, int hb, int c0, int c1, const SegOut &so) {
        const int g0 = hb * GB;                 // first query row of the block
        const int ng = min(GB, a.R - g0);

        // B operands of the logit MFMAs: q pieces 4*ks + kb of row
        // 16*nb + i16 of the block.
        uint4 qb[NB][KS];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int rr = 16 * nb + i16;
            const size_t qr = rr < ng ? qrow(a, b, kvh, g0 + rr) : 0;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                qb[nb][ks] = make_uint4(0, 0, 0, 0);
                if (rr < ng)
                    qb[nb][ks] = *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.q) + qr * ROWB +
                                                                   (4 * ks + kb) * 16);
            }
        }

        f32x4_v acc[NB][PVE];
        float m[NB], l[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int i = 0; i < PVE; ++i) acc[nb][i] = f32x4_v{0.f, 0.f, 0.f, 0.f};
            m[nb] = kNegInf;
            l[nb] = 0.f;
        }

        const char *kbase = static_cast<const char *>(a.k);
        const char *vbase = static_cast<const char *>(a.v);
        if constexpr (!PAGED) {
            const size_t seq = (size_t)(b * a.Hkv + kvh) * (size_t)a.T * ROWB;
            kbase += seq;
            vbase += seq;
        }

        // Paged: page ids of the range being streamed, staged in LDS so that
        // no K/V load waits on a dependent page-table read (ids outside the
        // pool become -1).  A range spans at most kMaxSplitPages pages.
        int p0 = 0;
        auto stage_pages = [&](int r0, int r1) {
            if constexpr (PAGED) {
                p0 = r0 >> a.page_shift;
                const int npg = r1 > r0 ? ((r1 - 1) >> a.page_shift) - p0 + 1 : 0;
                __syncthreads();
                for (int i = threadIdx.x; i < npg; i += 64 * WAVES) {
                    const int pg = a.page_table[(size_t)b * a.max_pages + p0 + i];
                    s_pages[i] = (unsigned)pg < (unsigned)a.num_pages ? pg : -1;
                }
                __syncthreads();
            }
        };

        // K/V pieces of one 32-token wave step (two 16-token tiles).
        struct Buf {
            uint4 k[2][KS];
            VP v[2][4];
            bool ok[2][4];
        };

        // sees(nb, t): query row 16*nb + i16 of the block attends to token
        // t (0..31) of the wave's step (false masks it, for the causal tail
        // of several queries).
        auto consume_step = [&](const Buf &f, auto sees) {
            float p[NB][2][4];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float s[2][4];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    f32x4_v c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) c = mfma_logits<DT>(f.k[h][ks], qb[nb][ks], c);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        s[h][r] = (f.ok[h][r] && sees(nb, 16 * h + 4 * kb + r)) ? c[r] * a.scale_log2 : kNegInf;
                }
                float mt = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                                 fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
                mt = fmaxf(mt, __shfl_xor(mt, 16));
                mt = fmaxf(mt, __shfl_xor(mt, 32));
                const float mn = fmaxf(m[nb], mt);
                const float mu = mn == kNegInf ? 0.f : mn;
                const float alpha = __builtin_amdgcn_exp2f(m[nb] - mu);
                float ps = 0.f;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        p[nb][h][r] = __builtin_amdgcn_exp2f(s[h][r] - mu);
                        ps += p[nb][h][r];
                    }
                l[nb] = l[nb] * alpha + ps;
                m[nb] = mn;
                // (skipped when no lane's max moved: alpha is then 1 exactly)
                if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
                    for (int i = 0; i < PVE; ++i) acc[nb][i] *= alpha;
                }
            }
            if constexpr (TRV) {
                // O^T (16 dims x 16 rows per block) += V^T (dims x 32 tokens)
                // . P^T (tokens x rows).  k slot 4h + r of lane (i16, kb) is
                // token 16h + 4kb + r on both operands: the B operand is the
                // lane's own probabilities, in a high and a low 16-bit part
                // (P = hi + lo to ~2^-16 relative), and the A operand comes
                // from two transposing reads of the wave's V tile.  acc[nb][dt]
                // then holds dims 16*dt + 4*kb .. +3 of row i16.
                unsigned char *wv = s_v[wave];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        *reinterpret_cast<VP *>(wv + (16 * h + 4 * kb + r) * VROW + VB * i16) = f.v[h][r];
                uint4 phi[NB], plo[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    uint32_t hi[4], lo[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = p[nb][e >> 1][2 * (e & 1)], y = p[nb][e >> 1][2 * (e & 1) + 1];
                        hi[e] = pack_p<DT>(x, y);
                        float hx, hy;
                        unpack_p<DT>(hi[e], hx, hy);
                        lo[e] = pack_p<DT>(x - hx, y - hy);
                    }
                    phi[nb] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                    plo[nb] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
                }
                const unsigned char *rd = wv + (4 * kb + (i16 >> 2)) * VROW + 8 * (i16 & 3);
#pragma unroll
                for (int dt = 0; dt < PVE; ++dt) {
                    const uint2 a0 = lds_read_tr16(rd + 32 * dt);
                    const uint2 a1 = lds_read_tr16(rd + 16 * VROW + 32 * dt);
                    const uint4 va = make_uint4(a0.x, a0.y, a1.x, a1.y);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) acc[nb][dt] = mfma_logits<DT>(va, phi[nb], acc[nb][dt]);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) acc[nb][dt] = mfma_logits<DT>(va, plo[nb], acc[nb][dt]);
                }
                return;
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float vf[PVE];
                    widen<DT>(f.v[h][r], vf);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int i = 0; i < PVE; ++i)
                            acc[nb][i] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[i], p[nb][h][r], acc[nb][i], 0, 0, 0);
                }
        };
        auto all_rows = [](int, int) { return true; };

        auto stream_range = [&](int r0, int r1) {
            auto row_offset = [&](int t, bool &ok) -> Off {
                ok = t < r1;
                const int tc = ok ? t : r1 - 1;        // clamped: always a valid token
                if constexpr (PAGED) {
                    int page = s_pages[(tc >> a.page_shift) - p0];
                    if (page < 0) { ok = false; page = 0; }
                    return (((size_t)page * a.Hkv + kvh) * a.page_size + (tc & (a.page_size - 1))) * ROWB;
                } else {
                    return (uint32_t)tc * (uint32_t)ROWB;
                }
            };

            // Pages of 16 tokens or more: a 16-token block (16-aligned, as every
            // range starts on a multiple of the tile) lies in one page, so one
            // page lookup serves the block's K and V rows.  The page is the
            // same for the whole wave, so the block's base address is kept in
            // scalar registers and each lane adds a fixed 32-bit offset -- the
            // same load form as the contiguous path.  A block past the range
            // end is redirected to the range's last block; its rows are read
            // but masked.
            constexpr bool block_pages = PG == 2;
            const uint32_t k_lane = (uint32_t)(i16 * ROWB + kb * 16);         // + 64 * ks
            const uint32_t v_lane = (uint32_t)(4 * kb * ROWB + i16 * VB);     // + ROWB * r
            auto block_base = [&](int t16, bool &page_ok) -> size_t {
                const int tcl = t16 < r1 ? t16 : ((r1 - 1) & ~15);
                int page = __builtin_amdgcn_readfirstlane(s_pages[(tcl >> a.page_shift) - p0]);
                page_ok = page >= 0;
                page = page_ok ? page : 0;
                return (((size_t)page * a.Hkv + kvh) * a.page_size + (tcl & (a.page_size - 1))) * ROWB;
            };

            auto load_step = [&](int base, Buf &f) {
                const int tb = base + wave * TOK;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int t16 = tb + 16 * h;
                    if constexpr (block_pages) {
                        bool pok;
                        const size_t bo = block_base(t16, pok);
                        const char *kblk = kbase + bo;
                        const char *vblk = vbase + bo;
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks)
                            f.k[h][ks] = load_piece<uint4>(kblk + (k_lane + (uint32_t)(64 * ks)));
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            f.ok[h][r] = pok && (t16 + 4 * kb + r < r1);
                            f.v[h][r] = load_piece<VP>(vblk + (v_lane + (uint32_t)(ROWB * r)));
                        }
                    } else {
                        bool okk;
                        const Off ko = row_offset(t16 + i16, okk);
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks)
                            f.k[h][ks] = load_piece<uint4>(kbase + (ko + (Off)((4 * ks + kb) * 16)));
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const Off vo = row_offset(t16 + 4 * kb + r, f.ok[h][r]);
                            f.v[h][r] = load_piece<VP>(vbase + (vo + (Off)(i16 * VB)));
                        }
                    }
                }
            };

            Buf fa, fb;
            load_step(r0, fa);
            for (int base = r0;; base += 2 * TILE) {
                load_step(base + TILE, fb);            // clamped past the end
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                consume_step(fa, all_rows);
                if (base + TILE >= r1) break;
                load_step(base + 2 * TILE, fa);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                consume_step(fb, all_rows);
                if (base + 2 * TILE >= r1) break;
            }
        };

        // Tokens every query row attends to are streamed by the main loop:
        // [c0, e1).  After it come the tokens some rows skip -- the causal
        // tail of several queries, or the appended token -- one at a time.
        int e1 = c1;
        int Tc = 0, tail0 = c1;
        if (a.append) {
            Tc = cached_len(a, b);
            e1 = c1 < Tc ? c1 : Tc;
        }
        if (a.causal) {
            Tc = cached_len(a, b);
            tail0 = max(c0, Tc - (a.nq - 1));
            e1 = min(e1, tail0);
        }

        if constexpr (PAGED) {
            // ranges of at most kMaxSplitPages pages: each ends on a page
            // boundary, so a start inside a page still fits the stage
            for (int r0 = c0, r1; r0 < e1; r0 = r1) {
                const long long e = ((long long)(r0 >> a.page_shift) + kMaxSplitPages) << a.page_shift;
                r1 = e < e1 ? (int)e : e1;
                stage_pages(r0, r1);
                if (STREAM) FD_MARK(a, 3 + 4 * so.ord);
                stream_range(r0, r1);
            }
        } else {
            if (c0 < e1) stream_range(c0, e1);
        }
        if (STREAM) FD_MARK(a, 4 + 4 * so.ord);

        // A few tokens (count <= 16) as the first tile of wave 0: lane i16
        // loads token i16's K row and lane (i16, kb) token 4*kb + r's V rows.
        // token_at(i, ok) gives token i's row offset from kb_ / vb_ (ok =
        // false: no such row); sees(i, row) tells whether a query row
        // attends to token i.  The other tile and waves are masked.
        auto fold_tokens = [&](const char *kb_, const char *vb_, int count, auto token_at, auto sees) {
            Buf f;
            bool kok;
            const size_t ko = token_at(i16 < count ? i16 : count - 1, kok);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    f.k[h][ks] = *reinterpret_cast<const uint4 *>(kb_ + ko + (4 * ks + kb) * 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ti = 4 * kb + r;
                bool vok;
                const size_t vo = token_at(ti < count ? ti : count - 1, vok);
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    f.v[h][r] = *reinterpret_cast<const VP *>(vb_ + vo + i16 * VB);
                f.ok[0][r] = wave == 0 && ti < count && vok;
                f.ok[1][r] = false;
            }
            consume_step(f, [&](int nb, int t) { return sees(t, g0 + 16 * nb + i16); });
        };

        if (a.causal && c1 > tail0) {
            // the causal tail: query row r (query r / G) sees tokens below
            // Tc - (nq - 1 - r / G)
            auto tail_token = [&](int i, bool &ok) -> size_t {
                const int t = tail0 + i;
                ok = true;
                if constexpr (PAGED) {
                    const int pg = a.page_table[(size_t)b * a.max_pages + (t >> a.page_shift)];
                    ok = (unsigned)pg < (unsigned)a.num_pages;
                    return (((size_t)(ok ? pg : 0) * a.Hkv + kvh) * a.page_size + (t & (a.page_size - 1))) * ROWB;
                } else {
                    return (size_t)t * ROWB;
                }
            };
            fold_tokens(kbase, vbase, c1 - tail0, tail_token,
                        [&](int i, int r) { return tail0 + i < Tc - (a.nq - 1 - r / a.G); });
        }

        if (a.append && c1 > Tc) {
            // the new token, read from the input rows
            const size_t nr = ((size_t)b * a.Hkv + kvh) * ROWB;
            fold_tokens(static_cast<const char *>(a.k_new) + nr, static_cast<const char *>(a.v_new) + nr, 1,
                        [](int, bool &ok) -> size_t { ok = true; return 0; },
                        [](int, int) { return true; });
            if (hb == 0) store_new_token<ROWB>(a, b, kvh, Tc);
        }

        // The four lanes of a head share m; their sums cover different tokens.
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            l[nb] += __shfl_xor(l[nb], 16);
            l[nb] += __shfl_xor(l[nb], 32);
        }

        __syncthreads();                               // sm is free (previous segment)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int i = 0; i < PVE; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (TRV) sm.o[wave][16 * nb + i16][16 * i + 4 * kb + r] = acc[nb][i][r];
                    else sm.o[wave][16 * nb + i16][PVE * (4 * kb + r) + i] = acc[nb][i][r];
                }
            if (kb == 0) { sm.m[wave][16 * nb + i16] = m[nb]; sm.l[wave][16 * nb + i16] = l[nb]; }
        }
        __syncthreads();
        finish_split<WAVES, GB, D>(a, sm, so, b, kvh, g0, ng);
    };

    if constexpr (STREAM) {
        __shared__ long long s_pref[kStreamMaxB + 1];
        drive_stream<64 * WAVES, D>(a, s_pref, GB, segment,
                                    [&](int b, int kvh, int hb, const SegOut &so, bool fence) {
                                        const int g0 = hb * GB;
                                        arrive_and_merge<WAVES, GB, D>(a, sm, so, b, kvh, g0,
                                                                       min(GB, a.R - g0), fence);
                                    });
    } else {
        const int split = blockIdx.x;
        const int kvh = blockIdx.y / a.head_blocks;
        const int hb = blockIdx.y - kvh * a.head_blocks;
        const int b = blockIdx.z;
        const int Tb = attended_len(a, b);
        const int c0 = split * a.chunk;
        const int c1 = min(c0 + a.chunk, Tb);
        const int g0 = hb * GB;
        if (a.n_splits > 1 && c0 >= Tb) {          // empty split: never counted or read
            if (a.fused && split == 0) write_empty_group<D>(a, b, kvh, g0, min(GB, a.R - g0));
            return;
        }
        segment(b, kvh, hb, c0, c1 > c0 ? c1 : c0, split_segment(a, b, kvh, hb, g0, split, Tb));
    }
}

template <int DT, int D, int NB>
hipError_t launch_nb(const SplitArgs &a, hipStream_t stream) {
    const dim3 grid = a.stream ? dim3(a.n_splits) : dim3(a.n_splits, a.Hkv * a.head_blocks, a.B);
    const int pg = !a.page_table ? 0 : (a.page_size >= 16 ? 2 : 1);
    if (a.stream) {
        if (pg == 2) hipLaunchKernelGGL((split_mfma<DT, D, 2, true, NB>), grid, dim3(256), 0, stream, a);
        else if (pg == 1) hipLaunchKernelGGL((split_mfma<DT, D, 1, true, NB>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((split_mfma<DT, D, 0, true, NB>), grid, dim3(256), 0, stream, a);
    } else {
        if (pg == 2) hipLaunchKernelGGL((split_mfma<DT, D, 2, false, NB>), grid, dim3(256), 0, stream, a);
        else if (pg == 1) hipLaunchKernelGGL((split_mfma<DT, D, 1, false, NB>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((split_mfma<DT, D, 0, false, NB>), grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_dim(const SplitArgs &a, hipStream_t stream) {
    return a.heads_per_block == 2 * kMfmaHeads ? launch_nb<DT, D, 2>(a, stream) : launch_nb<DT, D, 1>(a, stream);
}

template <int DT>
hipError_t launch_dtype(const SplitArgs &a, hipStream_t stream) {
    switch (a.D) {
    case 64: return launch_dim<DT, 64>(a, stream);
    case 128: return launch_dim<DT, 128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_split_mfma(const SplitArgs &a, int dtype, hipStream_t stream) {
    if (a.heads_per_block != kMfmaHeads && a.heads_per_block != 2 * kMfmaHeads) return hipErrorInvalidValue;
    switch (dtype) {
    case FD_F16: return launch_dtype<FD_F16>(a, stream);
    case FD_BF16: return launch_dtype<FD_BF16>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace fdk
