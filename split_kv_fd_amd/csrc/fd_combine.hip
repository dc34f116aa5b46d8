// Combine pass of flash decoding (tinyvolt "Kernel visualization: Flash
// Decoding", "Combine kernel"): the partials of every split are aligned to
// the global max and summed, and the result is divided once by the global
// normaliser.  Shift invariance of softmax makes this exact (zenaique
// explainer, interview answer on exactness).
//
// One 64-lane wavefront per (batch, query head), four per workgroup.  The
// global max and normaliser are wave reductions over the splits (lanes
// stride over splits); the weighted sum over splits runs with each lane
// owning D/64 output elements, reading the partial rows coalesced.  Split
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
    for (int s = lane; s < n; s += 64) L += __builtin_amdgcn_exp2f(pm[s] - mu) * pl[s];
    L = wave_sum(L);

    float acc[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[j] = 0.f;
    for (int s = 0; s < n; ++s) {
        const float w = __builtin_amdgcn_exp2f(pm[s] - mu);
        const float *row = po + (size_t)s * D + lane * DPL;
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[j] = fmaf(w, row[j], acc[j]);
    }

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
