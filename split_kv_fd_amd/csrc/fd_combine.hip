// Combine pass of flash decoding (tinyvolt "Kernel visualization: Flash
// Decoding", "Combine kernel"): the partials of every split are aligned to
// the global max and summed, and the result is divided once by the global
// normaliser.  Shift invariance of softmax makes this exact (zenaique
// explainer, interview answer on exactness).
//
// One 256-thread workgroup per (batch, query head).  Thread t owns four
// output elements (quad t % (D/4)) for the splits s = t / (D/4) (mod SG),
// SG = 256 / (D/4).  The partial rows of its first PRE splits are loaded
// together with the split maxima and sums, so a merge of up to PRE*SG
// splits costs one memory round trip; the global max and normaliser are
// workgroup reductions, and the SG partial sums of each quad are added in
// split-group order (deterministic).  Split maxima are in base-2 units (the
// split kernel folds log2(e) into the scale).  Splits that start past the
// tokens a row sees (the sequence's length; for causal queries fewer) may
// not have been written and are not read.
#include "fd_kernels.h"

namespace fdk {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309417f;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
    return x;
}

template <int D>
__global__ __launch_bounds__(256) void combine(CombineArgs a) {
    constexpr int NT = 256;
    constexpr int Q = D / 4;          // float4 quads per row
    constexpr int SG = NT / Q;        // split groups
    constexpr int PRE = 4;            // partial rows preloaded per thread
    constexpr int WCH = 2048;         // split weights staged per pass
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int q = t % Q, sg = t / Q;
    // partial row p = (b * Hkv + kv head) * R + query row; its output row is
    // (b * nq + query) * Hq + kv head * G + head of the group
    const int bh = blockIdx.x;
    const int b = bh / (a.Hkv * a.R);
    const int kvh = bh / a.R - b * a.Hkv;
    const int qr = bh - (bh / a.R) * a.R;
    const size_t orow = ((size_t)b * a.nq + qr / a.G) * a.Hq + (size_t)kvh * a.G + qr % a.G;

    int Tb = a.T;
    if (a.seq_lens) {
        Tb = a.seq_lens[b];
        Tb = Tb < 0 ? 0 : (Tb > a.T ? a.T : Tb);
    }
    Tb += a.append;                          // the appended token
    if (a.causal) {                          // this row's query sees fewer
        Tb -= a.nq - 1 - qr / a.G;
        Tb = Tb < 0 ? 0 : Tb;
    }
    int n = (Tb + a.chunk - 1) / a.chunk;   // splits that hold its tokens
    n = n < a.n_splits ? n : a.n_splits;

    const float *pm = a.part_m + (size_t)bh * a.n_splits;
    const float *pl = a.part_l + (size_t)bh * a.n_splits;
    const float4 *po = reinterpret_cast<const float4 *>(a.part_o + (size_t)bh * a.n_splits * D);

    // Issue the first partial rows together with the maxima.
    float4 pre[PRE];
#pragma unroll
    for (int j = 0; j < PRE; ++j) {
        const int s = sg + j * SG;
        pre[j] = s < n ? po[(size_t)s * Q + q] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float M = kNegInf;
    for (int s = t; s < n; s += NT) M = fmaxf(M, pm[s]);

    __shared__ float s_red[2][4];
    __shared__ float s_w[WCH];
    __shared__ float4 s_acc[SG][Q];
    M = wave_max(M);
    if (lane == 0) s_red[0][wave] = M;
    __syncthreads();
    M = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
    const float mu = M == kNegInf ? 0.f : M;

    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < n; s0 += WCH) {
        const int cnt = n - s0 < WCH ? n - s0 : WCH;
        if (s0 > 0) __syncthreads();          // previous weights consumed
        for (int i = t; i < cnt; i += NT) {
            const float w = __builtin_amdgcn_exp2f(pm[s0 + i] - mu);
            s_w[i] = w;
            L += w * pl[s0 + i];
        }
        __syncthreads();
        int s = sg;
        if (s0 == 0) {
#pragma unroll
            for (int j = 0; j < PRE; ++j, s += SG) {
                if (s < cnt) {
                    const float w = s_w[s];
                    acc.x = fmaf(w, pre[j].x, acc.x); acc.y = fmaf(w, pre[j].y, acc.y);
                    acc.z = fmaf(w, pre[j].z, acc.z); acc.w = fmaf(w, pre[j].w, acc.w);
                }
            }
        }
        for (; s < cnt; s += SG) {
            const float4 v = po[(size_t)(s0 + s) * Q + q];
            const float w = s_w[s];
            acc.x = fmaf(w, v.x, acc.x); acc.y = fmaf(w, v.y, acc.y);
            acc.z = fmaf(w, v.z, acc.z); acc.w = fmaf(w, v.w, acc.w);
        }
    }
    s_acc[sg][q] = acc;
    L = wave_sum(L);
    if (lane == 0) s_red[1][wave] = L;
    __syncthreads();
    L = (s_red[1][0] + s_red[1][1]) + (s_red[1][2] + s_red[1][3]);
    if (t < Q) {
        float4 r = s_acc[0][t];
        for (int g = 1; g < SG; ++g) {
            const float4 v = s_acc[g][t];
            r.x += v.x; r.y += v.y; r.z += v.z; r.w += v.w;
        }
        float4 o = L > 0.f ? make_float4(r.x / L, r.y / L, r.z / L, r.w / L) : make_float4(0.f, 0.f, 0.f, 0.f);
        reinterpret_cast<float4 *>(a.out + orow * D)[t] = o;
    }
    if (t == 0 && a.lse) a.lse[orow] = L > 0.f ? (M + log2f(L)) * kLn2 : kNegInf;
}

// The same merge with half a wave per partial row, eight rows per
// workgroup: for calls with many rows and few splits (the query-tiled
// kernel's), where a workgroup per row would idle most of its lanes and pay
// a workgroup's latency per row.  Lane i of a half owns elements D/32 * i ..
// of its row (one 16-byte load per split at D = 128); lane s of a half
// holds split s's max and sum.  The first PRE partial rows are loaded
// together with the maxima, so up to PRE splits cost one memory round
// trip.  Each lane adds its splits in order and the sums are xor-shuffle
// reductions within the half: results are deterministic.
template <int D>
__global__ __launch_bounds__(256) void combine_rows(CombineArgs a) {
    constexpr int LPR = 32;           // lanes per row
    constexpr int EPL = D / LPR;      // elements per lane
    constexpr int PRE = 16;
    typedef float vec_t __attribute__((ext_vector_type(EPL)));
    const int lane = threadIdx.x & 63;
    const int li = lane & (LPR - 1);
    const int base = lane & LPR;      // first lane of this half
    const long rows = (long)a.B * a.Hkv * a.R;
    const long bh = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2 + (lane >> 5);
    const bool live = bh < rows;      // a half past the last row idles (shuffles stay wave-wide)
    const long bq = live ? bh : 0;
    const int b = (int)(bq / ((long)a.Hkv * a.R));
    const int kvh = (int)(bq / a.R - (long)b * a.Hkv);
    const int qr = (int)(bq - (bq / a.R) * a.R);
    const size_t orow = ((size_t)b * a.nq + qr / a.G) * a.Hq + (size_t)kvh * a.G + qr % a.G;

    int Tb = a.T;
    if (a.seq_lens) {
        Tb = a.seq_lens[b];
        Tb = Tb < 0 ? 0 : (Tb > a.T ? a.T : Tb);
    }
    Tb += a.append;
    if (a.causal) {
        Tb -= a.nq - 1 - qr / a.G;
        Tb = Tb < 0 ? 0 : Tb;
    }
    const int chunk = a.dev_chunk ? *a.dev_chunk : a.chunk;
    int n = (Tb + chunk - 1) / chunk;
    n = n < a.n_splits ? n : a.n_splits;
    if (!live) n = 0;

    const float *pm = a.part_m + (size_t)bq * a.n_splits;
    const float *pl = a.part_l + (size_t)bq * a.n_splits;
    const vec_t *po = reinterpret_cast<const vec_t *>(a.part_o + (size_t)bq * a.n_splits * D) + li;

    vec_t pre[PRE];
#pragma unroll
    for (int j = 0; j < PRE; ++j) pre[j] = j < n ? po[(size_t)j * LPR] : vec_t{};
    float M = kNegInf;
    for (int s = li; s < n; s += LPR) M = fmaxf(M, pm[s]);
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float mu = M == kNegInf ? 0.f : M;

    float L = 0.f;
    vec_t acc{};
    for (int s0 = 0; s0 < n; s0 += LPR) {
        const int s = s0 + li;
        const float w = s < n ? __builtin_amdgcn_exp2f(pm[s] - mu) : 0.f;
        L += s < n ? w * pl[s] : 0.f;
        const int cnt = n - s0 < LPR ? n - s0 : LPR;
        int j = 0;
        if (s0 == 0) {
#pragma unroll
            for (; j < PRE; ++j)
                if (j < cnt) acc += __shfl(w, base + j) * pre[j];
        }
        for (; j < cnt; ++j) acc += __shfl(w, base + j) * po[(size_t)(s0 + j) * LPR];
    }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) L += __shfl_xor(L, off);
    if (!live) return;
    const vec_t o = L > 0.f ? acc / L : vec_t{};
    reinterpret_cast<vec_t *>(a.out + orow * D)[li] = o;
    if (li == 0 && a.lse) a.lse[orow] = L > 0.f ? (M + log2f(L)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t stream) {
    const long rows = (long)a.B * a.Hkv * a.R;
    if (a.per_wave) {
        const dim3 grid((unsigned)((rows + 7) / 8));
        switch (a.D) {
        case 64: hipLaunchKernelGGL(combine_rows<64>, grid, dim3(256), 0, stream, a); break;
        case 128: hipLaunchKernelGGL(combine_rows<128>, grid, dim3(256), 0, stream, a); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    const dim3 grid((unsigned)rows);
    switch (a.D) {
    case 64: hipLaunchKernelGGL(combine<64>, grid, dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(combine<128>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fdk
