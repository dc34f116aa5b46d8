// Query-tiled attention for many queries per sequence (the prefill phase)
// on the gfx950 matrix cores.
//
// The pages contrast the two phases (dupenodi guide "FlashDecoding and
// split-KV", "Concept" and "The big idea"): prefill attends with a whole
// block of queries and wants tiling over the query axis, decode has one
// query and wants the KV axis split.  This kernel is the query-tiled one:
// a workgroup owns kPrefillRows query rows of one (batch, kv head) -- the
// rows are (query, head of the GQA group) pairs, so every row of the tile
// reads the same K and V -- and walks the visible KV range in tiles of
// kPrefillTokens tokens with an online softmax (the same running max / sum
// / unnormalised accumulator as the split pass), then divides once.
//
// Per KV tile, staged in LDS by the whole workgroup (two buffers, the next
// tile's loads in flight while the current one is consumed):
//  * K rows as they are in memory (row stride padded by 16 bytes so the
//    16 lanes reading 16 rows hit distinct banks);
//  * V transposed, V^T[d][token], so that the value product can take 8
//    consecutive tokens of one dimension per lane.
// Per wave (16 rows) and tile (two 16-token halves):
//  * logits S^T = K Q^T with v_mfma_f32_16x16x32_{bf16,f16}: tokens on M,
//    query rows on N (the q pieces are the B operand, loaded once), so lane
//    (i16, kb) holds row i16's logits of tokens 4*kb .. 4*kb+3 of each half;
//  * online softmax in base 2 per row: max over the lane's 8 logits, then
//    across the four lanes of the row (xor 16, xor 32);
//  * values O^T += V^T P^T with the same MFMA: V^T rows from LDS as the A
//    operand, P^T from the lane's own probabilities as the B operand (k slot
//    8*kb + e is token 4*kb + e of the first half for e < 4, of the second
//    half for e >= 4, on both operands).  P goes in as a high and a low
//    16-bit part (P = hi + lo, two MFMAs), so its rounding stays near fp32:
//    a single bf16 P would spend the whole output tolerance.
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

// A finite fp32 value as the 16-bit storage type (round to nearest even),
// and back.
template <int DT>
__device__ __forceinline__ uint32_t to16(float x) {
    if constexpr (DT == FD_BF16) {
        const uint32_t u = __float_as_uint(x);
        return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    } else {
        return (uint32_t)__builtin_bit_cast(unsigned short, (_Float16)x);
    }
}

template <int DT>
__device__ __forceinline__ float from16(uint32_t h) {
    if constexpr (DT == FD_BF16) return __uint_as_float(h << 16);
    else return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
}

template <int DT, int D, bool PAGED>
__global__ __launch_bounds__(256, 2) void prefill(PrefillArgs a) {
    constexpr int ROWB = D * 2;              // bytes per K / V row
    constexpr int KS = D / 32;               // 32-wide k chunks of the logit product
    constexpr int DT16 = D / 16;             // 16-wide dimension tiles of the value product
    constexpr int PIECES = ROWB / 16;        // 16-byte pieces per row
    constexpr int NTOK = kPrefillTokens;     // tokens per KV tile
    constexpr int KSTR = ROWB + 16;          // LDS row stride of K (bytes)
    constexpr int VSTR = NTOK * 2 + 16;      // LDS row stride of V^T (bytes)
    static_assert(NTOK == 32 && kPrefillRows == 64, "the tile maps assume 32 tokens x 64 rows");
    static_assert(PIECES * 16 <= 256, "one (token pair, piece) per thread");

    __shared__ __align__(16) unsigned char sK[2][NTOK * KSTR];
    __shared__ __align__(16) unsigned char sV[2][D * VSTR];
    __shared__ int sOk[2][NTOK];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int i16 = lane & 15;
    const int kb = lane >> 4;

    const int tile = a.causal ? a.row_tiles - 1 - (int)blockIdx.x : (int)blockIdx.x;   // longest first
    const int kvh = blockIdx.y;
    const int b = blockIdx.z;
    const int r0 = tile * kPrefillRows;

    int Tb = a.seq_lens ? a.seq_lens[b] : a.T;
    Tb = Tb < 0 ? 0 : (Tb > a.T ? a.T : Tb);

    // This lane's query row, the tokens it sees, and its q pieces.
    const int rr = r0 + 16 * wave + i16;
    const bool row_ok = rr < a.R;
    const int qi = row_ok ? rr / a.G : 0;
    int lim = 0;
    if (row_ok) lim = a.causal ? Tb - (a.nq - 1 - qi) : Tb;
    lim = lim < 0 ? 0 : lim;
    const size_t qrow = ((size_t)b * a.nq + qi) * a.Hq + (size_t)kvh * a.G + (row_ok ? rr - qi * a.G : 0);
    uint4 qb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qb[ks] = row_ok ? *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.q) + qrow * ROWB +
                                                             (4 * ks + kb) * 16)
                        : make_uint4(0, 0, 0, 0);

    // Tokens the workgroup's rows see at most.
    const int r_last = min(r0 + kPrefillRows, a.R) - 1;
    int seen = a.causal ? Tb - (a.nq - 1 - r_last / a.G) : Tb;
    seen = seen < 0 ? 0 : seen;
    const int nt = (seen + NTOK - 1) / NTOK;

    // Loader: thread t moves tokens 2u, 2u+1 of the tile, piece p of each.
    const int u = t & 15;
    const int piece = t >> 4;
    const bool loader = piece < PIECES;
    uint4 k0 = make_uint4(0, 0, 0, 0), k1 = k0, v0 = k0, v1 = k0;
    int ok0 = 0, ok1 = 0;
    // row of token tt of the sequence (a real token: Tb >= 1 here); ok =
    // false for a padding token or a page outside the pool
    auto token_row = [&](int tt, int &ok) -> size_t {
        const int tc = tt < Tb ? tt : Tb - 1;
        ok = tt < Tb;
        if constexpr (PAGED) {
            int pg = a.page_table[(size_t)b * a.max_pages + (tc >> a.page_shift)];
            if ((unsigned)pg >= (unsigned)a.num_pages) { ok = 0; pg = 0; }
            return ((size_t)pg * a.Hkv + kvh) * a.page_size + (tc & (a.page_size - 1));
        } else {
            return ((size_t)b * a.Hkv + kvh) * a.T + tc;
        }
    };
    auto load_tile = [&](int j) {
        const size_t ra = token_row(j * NTOK + 2 * u, ok0);
        const size_t rb = token_row(j * NTOK + 2 * u + 1, ok1);
        if (loader) {
            const char *kp = static_cast<const char *>(a.k) + piece * 16;
            const char *vp = static_cast<const char *>(a.v) + piece * 16;
            k0 = *reinterpret_cast<const uint4 *>(kp + ra * ROWB);
            k1 = *reinterpret_cast<const uint4 *>(kp + rb * ROWB);
            v0 = *reinterpret_cast<const uint4 *>(vp + ra * ROWB);
            v1 = *reinterpret_cast<const uint4 *>(vp + rb * ROWB);
        }
    };
    auto store_tile = [&](int buf) {
        if (!loader) return;
        *reinterpret_cast<uint4 *>(&sK[buf][(2 * u) * KSTR + piece * 16]) = k0;
        *reinterpret_cast<uint4 *>(&sK[buf][(2 * u + 1) * KSTR + piece * 16]) = k1;
        // V^T: dimension 8*piece + e, tokens 2u and 2u+1 packed in one word
        const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w};
        const uint32_t w1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<uint32_t *>(&sV[buf][(8 * piece + 2 * i) * VSTR + 4 * u]) =
                (w0[i] & 0xffffu) | (w1[i] << 16);
            *reinterpret_cast<uint32_t *>(&sV[buf][(8 * piece + 2 * i + 1) * VSTR + 4 * u]) =
                (w0[i] >> 16) | (w1[i] & 0xffff0000u);
        }
        if (piece == 0) {
            sOk[buf][2 * u] = ok0;
            sOk[buf][2 * u + 1] = ok1;
        }
    };

    f32x4_v acc[DT16];
#pragma unroll
    for (int dt = 0; dt < DT16; ++dt) acc[dt] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, l = 0.f;

    if (nt > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();
    for (int j = 0; j < nt; ++j) {
        const int buf = j & 1;
        if (j + 1 < nt) load_tile(j + 1);            // in flight while this tile is consumed

        float s[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f32x4_v c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint4 kp = *reinterpret_cast<const uint4 *>(&sK[buf][(16 * h + i16) * KSTR + (4 * ks + kb) * 16]);
                c = mfma<DT>(kp, qb[ks], c);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tk = 16 * h + 4 * kb + r;
                const bool ok = sOk[buf][tk] && (j * NTOK + tk < lim);
                s[h][r] = ok ? c[r] * a.scale_log2 : kNegInf;
            }
        }
        float mt = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m, mt);
        const float mu = mn == kNegInf ? 0.f : mn;
        const float alpha = __builtin_amdgcn_exp2f(m - mu);
        float p[8];
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(s[e >> 2][e & 3] - mu);
            ps += p[e];
        }
        l = l * alpha + ps;
        m = mn;
        // P^T as the B operand, in two 16-bit parts
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            hi[e] = to16<DT>(p[e]);
            lo[e] = to16<DT>(p[e] - from16<DT>(hi[e]));
        }
        const uint4 phi = make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16),
                                     hi[6] | (hi[7] << 16));
        const uint4 plo = make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16),
                                     lo[6] | (lo[7] << 16));
#pragma unroll
        for (int dt = 0; dt < DT16; ++dt) {
            const unsigned char *vrow = &sV[buf][(16 * dt + i16) * VSTR];
            const uint2 v0 = *reinterpret_cast<const uint2 *>(vrow + 8 * kb);
            const uint2 v1 = *reinterpret_cast<const uint2 *>(vrow + 32 + 8 * kb);
            const uint4 va = make_uint4(v0.x, v0.y, v1.x, v1.y);
            acc[dt] *= alpha;
            acc[dt] = mfma<DT>(va, phi, acc[dt]);
            acc[dt] = mfma<DT>(va, plo, acc[dt]);
        }

        if (j + 1 < nt) store_tile(buf ^ 1);
        __syncthreads();
    }

    // The four lanes of a row share m; their sums cover different tokens.
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (!row_ok) return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT16; ++dt) {
        const f32x4_v o = acc[dt] * inv;
        *reinterpret_cast<float4 *>(a.out + qrow * D + 16 * dt + 4 * kb) = make_float4(o[0], o[1], o[2], o[3]);
    }
    if (kb == 0 && a.lse) a.lse[qrow] = l > 0.f ? (m + log2f(l)) * kLn2 : kNegInf;
}

template <int DT, int D>
hipError_t launch_dim(const PrefillArgs &a, hipStream_t stream) {
    const dim3 grid(a.row_tiles, a.Hkv, a.B);
    if (a.page_table) hipLaunchKernelGGL((prefill<DT, D, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((prefill<DT, D, false>), grid, dim3(256), 0, stream, a);
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
