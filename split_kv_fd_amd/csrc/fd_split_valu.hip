// Split pass of flash decoding on the vector ALUs of gfx950.
//
// One workgroup per (batch, kv head, head block, split) streams its chunk of
// K and V once, for every query head of its GQA group, and leaves an
// unnormalised partial with its running max and sum (tinyvolt "Kernel
// visualization: Flash Decoding", "Visualizing operations in a single
// block"; the combine kernel merges the partials).
//
// How the work maps onto CDNA4 instead of the pages' one-thread softmax:
//  * a token row of K or V (D elements) is read as 16-byte pieces by LPR
//    consecutive lanes, so one load instruction fetches R = 64/LPR whole
//    rows (1 KiB contiguous for D=128 at 2 bytes per element);
//  * the q.k partial sums of a row are reduced across its LPR lanes with
//    DPP row permutes (quad swaps, half-row and row mirrors), which leave
//    the same bits in every lane of the row;
//  * every row of every wave runs its own online softmax over the tokens it
//    sees (running max m, sum l, unnormalised accumulator o), in base 2 with
//    log2(e) folded into the scale; rows and waves are merged at the end by
//    the same log-sum-exp rule the combine uses, so no per-token cross-row
//    traffic is needed;
//  * the next step's K/V pieces are loaded into registers before the
//    current step is consumed, so each wave keeps two steps in flight.
// Tokens past the chunk end are read from a clamped, valid address and get
// a -inf logit, which keeps every load unconditional.
#include <type_traits>

#include "fd_epilogue.h"

namespace fdk {
namespace {

typedef _Float16 half2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_v __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LPR (8 or 16) lanes; all lanes of a group end
// with identical bits (each step adds a commuted pair).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
    x += dpp_mov<0x141>(x);   // row_half_mirror: the other quad of 8 lanes
    if constexpr (LPR == 16)
        x += dpp_mov<0x140>(x);   // row_mirror: the other half of 16 lanes
    return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// q.k over one 16-byte piece, accumulated in fp32.  Products of two f16 or
// two bf16 values are exact in fp32.
template <int DT>
__device__ __forceinline__ float dot_piece(const uint4 &q, const uint4 &k, float acc) {
    if constexpr (DT == FD_F32) {
        acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
        acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
        acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
        acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
    } else if constexpr (DT == FD_F16) {
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_v, q.x), __builtin_bit_cast(half2_v, k.x), acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_v, q.y), __builtin_bit_cast(half2_v, k.y), acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_v, q.z), __builtin_bit_cast(half2_v, k.z), acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_v, q.w), __builtin_bit_cast(half2_v, k.w), acc, false);
    } else {
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_v, q.x), __builtin_bit_cast(bf162_v, k.x), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_v, q.y), __builtin_bit_cast(bf162_v, k.y), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_v, q.z), __builtin_bit_cast(bf162_v, k.z), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_v, q.w), __builtin_bit_cast(bf162_v, k.w), acc, false);
    }
    return acc;
}

__device__ __forceinline__ float f16_lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

// The elements of one 16-byte piece as fp32 (exact widening).
template <int DT>
__device__ __forceinline__ void widen(const uint4 &p, float *f) {
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
    if constexpr (DT == FD_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
    } else if constexpr (DT == FD_F16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[2 * i] = f16_lo(w[i]); f[2 * i + 1] = f16_hi(w[i]); }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
}

typedef unsigned int u32x4_v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load16(const char *p) {
#if FD_NT_LOADS
    const u32x4_v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_v *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
#else
    return *reinterpret_cast<const uint4 *>(p);
#endif
}

// STREAM: balanced stream mode (ragged batches), else one workgroup per
// (batch, kv head, head block, split).
template <int DT, int D, int GB, bool PAGED, bool STREAM>
__global__ __launch_bounds__(256) void split_valu(SplitArgs a) {
    constexpr int EB = DT == FD_F32 ? 4 : 2;
    using S = ValuShape<EB, D, GB>;
    constexpr int LPR = S::LPR, VEC = S::VEC, EPC = S::EPC, EPT = S::EPT;
    constexpr int R = S::R, U = S::U, TW = S::TW, TILE = S::TILE, WAVES = S::WAVES;
    constexpr int ROWB = S::ROWB;
    static_assert(WAVES * 64 == 256, "launch bounds assume 256 threads");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
    const int row = lane / LPR;
    const int sub = lane % LPR;

    __shared__ int s_pages[PAGED ? kMaxSplitPages : 1];
    __shared__ EpilogueLds<WAVES, GB, D> sm;

    // One segment: tokens [c0, c1) of row (b, kvh, hb) into `so`.
    auto segment = [&](int b, int kvh, int hb, int c0, int c1, const SegOut &so) {
        const int g0 = hb * GB;                     // first query row of the block
        const int ng = min(GB, a.R - g0);          // valid query rows in this block

        // This lane's pieces of the query rows (raw storage words).
        uint4 qv[GB][VEC];
#pragma unroll
        for (int g = 0; g < GB; ++g) {
            const size_t qr = g < ng ? qrow(a, b, kvh, g0 + g) : 0;
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                qv[g][v] = make_uint4(0, 0, 0, 0);
                if (g < ng)
                    qv[g][v] = *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.q) + qr * ROWB +
                                                                 (v * LPR + sub) * 16);
            }
        }

        float m[GB], l[GB], o[GB][EPT];
#pragma unroll
        for (int g = 0; g < GB; ++g) {
            m[g] = kNegInf;
            l[g] = 0.f;
#pragma unroll
            for (int e = 0; e < EPT; ++e) o[g][e] = 0.f;
        }

        const char *kb = static_cast<const char *>(a.k);
        const char *vb = static_cast<const char *>(a.v);
        if constexpr (!PAGED) {
            const size_t seq = (size_t)(b * a.Hkv + kvh) * (size_t)a.T * ROWB;
            kb += seq;
            vb += seq;
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

        // rows_ok(u, g): query row g attends to this lane's token u (false
        // masks it, for the causal tail of several queries).
        auto consume_step = [&](const uint4 (&kr)[U][VEC], const uint4 (&vr)[U][VEC], const bool (&ok)[U],
                                auto rows_ok) {
            float s[U][GB];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int g = 0; g < GB; ++g) {
                    float acc = 0.f;
#pragma unroll
                    for (int v = 0; v < VEC; ++v) acc = dot_piece<DT>(qv[g][v], kr[u][v], acc);
                    acc = row_sum<LPR>(acc) * a.scale_log2;
                    s[u][g] = (ok[u] && rows_ok(u, g)) ? acc : kNegInf;
                }
            float vf[U][EPT];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int v = 0; v < VEC; ++v) widen<DT>(vr[u][v], &vf[u][v * EPC]);
#pragma unroll
            for (int g = 0; g < GB; ++g) {
                float mt = s[0][g];
#pragma unroll
                for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[u][g]);
                const float mn = fmaxf(m[g], mt);
                const float mu = mn == kNegInf ? 0.f : mn;
                const float alpha = exp2_fast(m[g] - mu);
                float p[U];
                float ps = 0.f;
#pragma unroll
                for (int u = 0; u < U; ++u) { p[u] = exp2_fast(s[u][g] - mu); ps += p[u]; }
                l[g] = l[g] * alpha + ps;
#pragma unroll
                for (int e = 0; e < EPT; ++e) {
                    float acc = o[g][e] * alpha;
#pragma unroll
                    for (int u = 0; u < U; ++u) acc = fmaf(p[u], vf[u][e], acc);
                    o[g][e] = acc;
                }
                m[g] = mn;
            }
        };

        auto all_rows = [](int, int) { return true; };

        auto stream_range = [&](int r0, int r1) {
            // Byte offset of token t's row and whether the token is real.  A
            // contiguous (batch, kv head) slice is below 4 GiB (checked on the
            // host), so its offsets are 32-bit: the loads then take a scalar
            // base address plus one vector register.
            using Off = typename std::conditional<PAGED, size_t, uint32_t>::type;
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

            auto load_step = [&](int base, uint4 (&kr)[U][VEC], uint4 (&vr)[U][VEC], bool (&ok)[U]) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const Off off = row_offset(base + wave * TW + u * R + row, ok[u]);
#pragma unroll
                    for (int v = 0; v < VEC; ++v) {
                        kr[u][v] = load16(kb + (off + (Off)((v * LPR + sub) * 16)));
                        vr[u][v] = load16(vb + (off + (Off)((v * LPR + sub) * 16)));
                    }
                }
            };

            // Two register buffers used in turn: while one step is consumed
            // the next one is in flight.  The fence keeps each prefetch where
            // it is issued (otherwise the compiler sinks every load next to
            // its first use one step later), and the scheduling barrier stops
            // the consumer's arithmetic from being hoisted above it.
            uint4 ka[U][VEC], va[U][VEC], kb2[U][VEC], vb2[U][VEC];
            bool oka[U], okb[U];
            load_step(r0, ka, va, oka);
            for (int base = r0;; base += 2 * TILE) {
                load_step(base + TILE, kb2, vb2, okb);   // clamped past the end
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                consume_step(ka, va, oka, all_rows);
                if (base + TILE >= r1) break;
                load_step(base + 2 * TILE, ka, va, oka);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                consume_step(kb2, vb2, okb, all_rows);
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
                stream_range(r0, r1);
            }
        } else {
            if (c0 < e1) stream_range(c0, e1);
        }

        // A few tokens (count <= TILE) in the slots of one step: slot i =
        // wave * TW + u * R + row, as in the main loop.  token_at(i, ok) gives
        // token i's row offset from kb_ / vb_ (ok = false: no such row);
        // sees(i, row) tells whether a query row attends to token i.
        auto fold_tokens = [&](const char *kb_, const char *vb_, int count, auto token_at, auto sees) {
            uint4 kr[U][VEC], vr[U][VEC];
            bool ok[U];
            int ti[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                ti[u] = wave * TW + u * R + row;
                bool tok;
                const size_t off = token_at(ti[u] < count ? ti[u] : count - 1, tok);
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    kr[u][v] = *reinterpret_cast<const uint4 *>(kb_ + off + (v * LPR + sub) * 16);
                    vr[u][v] = *reinterpret_cast<const uint4 *>(vb_ + off + (v * LPR + sub) * 16);
                }
                ok[u] = ti[u] < count && tok;
            }
            consume_step(kr, vr, ok, [&](int u, int g) { return sees(ti[u], g0 + g); });
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
            fold_tokens(kb, vb, c1 - tail0, tail_token,
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

        // Merge the rows of this wave (log-sum-exp, rows LPR, 2*LPR, ... apart).
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
            for (int g = 0; g < GB; ++g) {
                const float m2 = __shfl_xor(m[g], off);
                const float l2 = __shfl_xor(l[g], off);
                const float mn = fmaxf(m[g], m2);
                const float mu = mn == kNegInf ? 0.f : mn;
                const float a1 = exp2_fast(m[g] - mu), a2 = exp2_fast(m2 - mu);
                l[g] = l[g] * a1 + l2 * a2;
#pragma unroll
                for (int e = 0; e < EPT; ++e) {
                    const float o2 = __shfl_xor(o[g][e], off);
                    o[g][e] = o[g][e] * a1 + o2 * a2;
                }
                m[g] = mn;
            }
        }

        // Merge the waves through LDS and finish the segment.
        __syncthreads();                               // sm is free (previous segment)
        if (row == 0) {
#pragma unroll
            for (int g = 0; g < GB; ++g) {
#pragma unroll
                for (int v = 0; v < VEC; ++v)
#pragma unroll
                    for (int j = 0; j < EPC; ++j)
                        sm.o[wave][g][(v * LPR + sub) * EPC + j] = o[g][v * EPC + j];
                if (sub == 0) { sm.m[wave][g] = m[g]; sm.l[wave][g] = l[g]; }
            }
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

template <int DT, int D, int GB, bool PAGED>
hipError_t launch_instance(const SplitArgs &a, hipStream_t stream) {
    if (a.stream) {
        hipLaunchKernelGGL((split_valu<DT, D, GB, PAGED, true>), dim3(a.n_splits), dim3(256), 0, stream, a);
    } else {
        const dim3 grid(a.n_splits, a.Hkv * a.head_blocks, a.B);
        hipLaunchKernelGGL((split_valu<DT, D, GB, PAGED, false>), grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

template <int DT, int D, int GB>
hipError_t launch_paged(const SplitArgs &a, hipStream_t s) {
    return a.page_table ? launch_instance<DT, D, GB, true>(a, s)
                        : launch_instance<DT, D, GB, false>(a, s);
}

template <int DT, int D>
hipError_t launch_heads(const SplitArgs &a, hipStream_t s) {
    switch (a.heads_per_block) {
    case 1: return launch_paged<DT, D, 1>(a, s);
    case 2: return launch_paged<DT, D, 2>(a, s);
    case 4: return launch_paged<DT, D, 4>(a, s);
    case 8: return launch_paged<DT, D, 8>(a, s);
    default: return hipErrorInvalidValue;
    }
}

template <int DT>
hipError_t launch_dim(const SplitArgs &a, hipStream_t s) {
    switch (a.D) {
    case 64: return launch_heads<DT, 64>(a, s);
    case 128: return launch_heads<DT, 128>(a, s);
    default: return hipErrorInvalidValue;
    }
}

template <int EB, int D>
int tile_of(int gb) {
    switch (gb) {
    case 1: return ValuShape<EB, D, 1>::TILE;
    case 2: return ValuShape<EB, D, 2>::TILE;
    case 4: return ValuShape<EB, D, 4>::TILE;
    case 8: return ValuShape<EB, D, 8>::TILE;
    default: return 0;
    }
}

}  // namespace

int valu_tile(int dtype, int D, int gb) {
    const bool f32 = dtype == FD_F32;
    if (D == 64) return f32 ? tile_of<4, 64>(gb) : tile_of<2, 64>(gb);
    if (D == 128) return f32 ? tile_of<4, 128>(gb) : tile_of<2, 128>(gb);
    return 0;
}

hipError_t launch_split_valu(const SplitArgs &a, int dtype, hipStream_t stream) {
    switch (dtype) {
    case FD_F32: return launch_dim<FD_F32>(a, stream);
    case FD_F16: return launch_dim<FD_F16>(a, stream);
    case FD_BF16: return launch_dim<FD_BF16>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace fdk
