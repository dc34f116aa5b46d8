// Combine pass of flash decoding (tinyvolt "Kernel visualization: Flash
// Decoding", "Combine kernel"): the partials of every split are aligned to
// the global max and summed, and the result is divided once by the global
// normaliser.  Shift invariance of softmax makes this exact (zenaique
// explainer, interview answer on exactness).
//
// One 64-lane wavefront per (batch, query head), four per workgroup.  The
// global max and normaliser are wave reductions over the splits (lanes
// stride over splits); the weighted sum over splits runs with each lane
// owning D/64 output elements, reading eight partial rows at a time so the
// loop is not bound by one memory round trip per split.  Split
// maxima are in base-2 units (the split kernel folds log2(e) into the
// scale).  Splits that start past a sequence's length were never written
// and are not read.
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
    constexpr int DPL = D / 64;   // output elements per lane
    constexpr int UNR = 8;        // partial rows in flight per lane
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (bh >= a.B * a.Hq) return;   // whole wave exits together
    const int b = bh / a.Hq;

    int Tb = a.T;
    if (a.seq_lens) {
        Tb = a.seq_lens[b];
        Tb = Tb < 0 ? 0 : (Tb > a.T ? a.T : Tb);
    }
    int n = (Tb + a.chunk - 1) / a.chunk;   // splits that hold tokens
    n = n < a.n_splits ? n : a.n_splits;

    const float *pm = a.part_m + (size_t)bh * a.n_splits;
    const float *pl = a.part_l + (size_t)bh * a.n_splits;
    const float *po = a.part_o + (size_t)bh * a.n_splits * D;

    float M = kNegInf;
    for (int s = lane; s < n; s += 64) M = fmaxf(M, pm[s]);
    M = wave_max(M);
    const float mu = M == kNegInf ? 0.f : M;

    float L = 0.f;
    float acc[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[j] = 0.f;
    // Lanes hold the weights of 64 splits at a time; each weight is
    // broadcast while UNR partial rows are read at once.
    for (int s0 = 0; s0 < n; s0 += 64) {
        const int s = s0 + lane;
        const float w = s < n ? __builtin_amdgcn_exp2f(pm[s] - mu) : 0.f;
        if (s < n) L += w * pl[s];
        const int cnt = n - s0 < 64 ? n - s0 : 64;
        for (int j0 = 0; j0 < cnt; j0 += UNR) {
            float v[UNR][DPL], wj[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const bool in = j0 + u < cnt;
                wj[u] = __shfl(w, j0 + u < 64 ? j0 + u : 63);
                const float *row = po + (size_t)(s0 + (in ? j0 + u : 0)) * D + lane * DPL;
#pragma unroll
                for (int j = 0; j < DPL; ++j) v[u][j] = in ? row[j] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u)
#pragma unroll
                for (int j = 0; j < DPL; ++j) acc[j] = fmaf(j0 + u < cnt ? wj[u] : 0.f, v[u][j], acc[j]);
        }
    }
    L = wave_sum(L);

    float *o = a.out + (size_t)bh * D + lane * DPL;
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[j] = L > 0.f ? acc[j] / L : 0.f;
    if (lane == 0 && a.lse) a.lse[bh] = L > 0.f ? (M + log2f(L)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t stream) {
    const int rows = a.B * a.Hq;
    const dim3 grid((rows + 3) / 4);
    switch (a.D) {
    case 64: hipLaunchKernelGGL(combine<64>, grid, dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(combine<128>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fdk
