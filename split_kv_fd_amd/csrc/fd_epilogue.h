// Device code shared by the split kernels: merging the per-wave softmax
// states of one workgroup, writing a split's partial (or the final result
// when there is a single split), and -- in the fused mode -- letting the
// last workgroup of a (batch, kv head, head block) merge all of its splits.
//
// The merge rule is the combine of tinyvolt's "Combine kernel" section:
// align every partial to the largest running max, sum the rescaled
// normalisers and accumulators, divide once.  Maxima are in base-2 units.
#pragma once

#include "fd_kernels.h"

namespace fdk {

constexpr float kEpNegInf = -__builtin_inff();
constexpr float kEpLn2 = 0.693147180559945309417f;

__device__ __forceinline__ float ep_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Count this workgroup's arrival at its group's counter.  The counter holds
// (call epoch << 32 | arrivals); a value left by any other call (another
// epoch) restarts the count, so the workspace needs no clearing between
// calls.  Returns true for the workgroup that completes the group.  The loop
// ends: every failed exchange means another workgroup's exchange succeeded.
//
// Ordering.  A device-scope release here would write back the whole L2 of
// the XCD for every workgroup (about 1.7 us each, serialised), which costs
// more than the separate combine launch it replaces.  Instead the partials
// are written and read only with device-coherent (sc1) accesses, which go to
// the coherent level instead of a per-XCD L2 copy; every thread waits for
// its stores to complete (vmcnt 0) before the barrier, so all partials of
// the workgroup are at the coherent level before this exchange is issued,
// and the last workgroup issues its coherent loads only after the exchange
// that completed the count has returned.
__device__ __forceinline__ bool arrive_last(unsigned long long *cnt, unsigned epoch, int n_active) {
    unsigned long long old = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned long long next;
    for (;;) {
        next = ((unsigned)(old >> 32) == epoch) ? old + 1ull
                                                 : (((unsigned long long)epoch << 32) | 1ull);
        if (__hip_atomic_compare_exchange_strong(cnt, &old, next, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
            break;
    }
    return (unsigned)(next & 0xffffffffull) == (unsigned)n_active;
}

// Device-coherent accesses of the partials in fused mode.
__device__ __forceinline__ void st_agent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float ld_agent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Largest heads x splits one fused merge handles (the planner keeps fused
// plans within it).
constexpr int kMergeMaxPairs = (int)kMergeMaxPairsHost;

// LDS the epilogue works in: per-wave states, then the fused merge's split
// maxima / weights, sums and per-split-group partial rows.
template <int WAVES, int GB, int D>
struct EpilogueLds {
    float o[WAVES][GB][D];
    float m[WAVES][GB];
    float l[WAVES][GB];
    float gm[GB];                  // merge: global max of each head
    float gl[GB];                  // merge: global normaliser of each head
    float w[kMergeMaxPairs];       // merge: split maxima, then weights
    float sl[kMergeMaxPairs];      // merge: split sums
    float4 red[WAVES * 64];        // merge: per split-group partial rows
    int last;
};

// A sequence with no tokens: out = 0 and lse = -inf for the block's heads.
// In fused mode no split of such a sequence reaches the merge, so split 0
// writes this instead.
template <int D>
__device__ void write_empty_group(const SplitArgs &a, int b, int h0, int ng) {
    for (int idx = threadIdx.x; idx < ng * D; idx += blockDim.x) {
        const int g = idx / D, d = idx - (idx / D) * D;
        const int bh = b * a.Hq + h0 + g;
        a.out[(size_t)bh * D + d] = 0.f;
        if (d == 0 && a.lse) a.lse[bh] = kEpNegInf;
    }
}

// Splits that hold tokens of a sequence of length Tb.
__device__ __forceinline__ int active_splits(const SplitArgs &a, int Tb) {
    const int n = (Tb + a.chunk - 1) / a.chunk;
    return n < a.n_splits ? n : a.n_splits;
}

// Merge the last workgroup's group: for every valid head g of the block,
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the n active
// splits, read back from the workspace.  The loads of the split maxima and
// sums and of each thread's first PRE partial rows are issued together, so
// a merge of up to PRE*SG splits costs one memory round trip.  Thread t owns
// one (head, float4 quad) pair and every SG-th split of it; sums run in
// split order within a thread and in split-group order across threads
// (deterministic).  ng * n <= kMergeMaxPairs.
template <int WAVES, int GB, int D>
__device__ void combine_group(const SplitArgs &a, EpilogueLds<WAVES, GB, D> &sm, int b, int h0, int ng,
                              int n) {
    constexpr int NT = WAVES * 64;
    constexpr int Q = D / 4;
    constexpr int PRE = 8;
    constexpr int MLR = kMergeMaxPairs / NT;            // maxima/sums per thread
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int nml = ng * n;
    const int pairs = ng * Q;
    int SG = 1;                                         // split groups per pair:
    while (SG * 2 * pairs <= NT) SG *= 2;               // a power of two, so NT % SG == 0
    const int per_pass = NT / SG;                       // pairs per pass

    float mr[MLR], lr[MLR];
#pragma unroll
    for (int k = 0; k < MLR; ++k) {
        const int i = t + k * NT;
        mr[k] = kEpNegInf;
        lr[k] = 0.f;
        if (i < nml) {
            const int g = i / n, s = i - (i / n) * n;
            const size_t row = (size_t)(b * a.Hq + h0 + g) * a.n_splits + s;
            mr[k] = ld_agent(a.part_m + row);
            lr[k] = ld_agent(a.part_l + row);
        }
    }
    for (int p0 = 0; p0 < pairs; p0 += per_pass) {
        const int p = p0 + t / SG, sg = t - (t / SG) * SG;
        const bool active = p < pairs;
        const int g = active ? p / Q : 0, q = active ? p - (p / Q) * Q : 0;
        const int bh = b * a.Hq + h0 + g;
        const float *po = a.part_o + (size_t)bh * a.n_splits * D + 4 * q;
        float4 pre[PRE];
#pragma unroll
        for (int j = 0; j < PRE; ++j) {
            const int s = sg + j * SG;
            pre[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (active && s < n) {
                const float *src = po + (size_t)s * D;
                pre[j] = make_float4(ld_agent(src), ld_agent(src + 1), ld_agent(src + 2), ld_agent(src + 3));
            }
        }
        if (p0 == 0) {
            // global max, weights and normaliser of each head (one wave per head)
#pragma unroll
            for (int k = 0; k < MLR; ++k) {
                const int i = t + k * NT;
                if (i < nml) { sm.w[i] = mr[k]; sm.sl[i] = lr[k]; }
            }
            __syncthreads();
            for (int g2 = wave; g2 < ng; g2 += WAVES) {
                float M = kEpNegInf;
                for (int s2 = lane; s2 < n; s2 += 64) M = fmaxf(M, sm.w[g2 * n + s2]);
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
                const float mu = M == kEpNegInf ? 0.f : M;
                float L = 0.f;
                for (int s2 = lane; s2 < n; s2 += 64) {
                    const float c = ep_exp2(sm.w[g2 * n + s2] - mu);
                    sm.w[g2 * n + s2] = c;
                    L = fmaf(c, sm.sl[g2 * n + s2], L);
                }
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) L += __shfl_xor(L, off);
                if (lane == 0) { sm.gm[g2] = M; sm.gl[g2] = L; }
            }
            __syncthreads();
        }
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (active) {
            const float *wg = sm.w + g * n;
            int s = sg;
#pragma unroll
            for (int j = 0; j < PRE; ++j, s += SG) {
                if (s < n) {
                    const float c = wg[s];
                    acc.x = fmaf(c, pre[j].x, acc.x); acc.y = fmaf(c, pre[j].y, acc.y);
                    acc.z = fmaf(c, pre[j].z, acc.z); acc.w = fmaf(c, pre[j].w, acc.w);
                }
            }
            for (; s < n; s += SG) {
                const float *src = po + (size_t)s * D;
                const float c = wg[s];
                acc.x = fmaf(c, ld_agent(src), acc.x); acc.y = fmaf(c, ld_agent(src + 1), acc.y);
                acc.z = fmaf(c, ld_agent(src + 2), acc.z); acc.w = fmaf(c, ld_agent(src + 3), acc.w);
            }
        }
        sm.red[sg * per_pass + (t / SG)] = acc;
        __syncthreads();
        if (active && sg == 0) {
            float4 r = sm.red[t / SG];
            for (int k2 = 1; k2 < SG; ++k2) {
                const float4 v = sm.red[k2 * per_pass + t / SG];
                r.x += v.x; r.y += v.y; r.z += v.z; r.w += v.w;
            }
            const float L = sm.gl[g];
            const float4 o = L > 0.f ? make_float4(r.x / L, r.y / L, r.z / L, r.w / L)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
            reinterpret_cast<float4 *>(a.out + (size_t)bh * D)[q] = o;
            if (q == 0 && a.lse) a.lse[bh] = L > 0.f ? (sm.gm[g] + log2f(L)) * kEpLn2 : kEpNegInf;
        }
        __syncthreads();
    }
}

// Called by every thread after sm.o / sm.m / sm.l hold each wave's state
// (the caller has synchronised).  Writes this split's result and, in fused
// mode, completes the group when this workgroup arrives last.
template <int WAVES, int GB, int D>
__device__ void finish_split(const SplitArgs &a, EpilogueLds<WAVES, GB, D> &sm, int b, int kvh, int hb,
                             int split, int h0, int ng, int Tb) {
    constexpr int NT = WAVES * 64;
    for (int idx = threadIdx.x; idx < ng * D; idx += NT) {
        const int g = idx / D, d = idx - (idx / D) * D;
        float M = sm.m[0][g];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) M = fmaxf(M, sm.m[w][g]);
        const float mu = M == kEpNegInf ? 0.f : M;
        float acc = 0.f, L = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float c = ep_exp2(sm.m[w][g] - mu);
            acc += c * sm.o[w][g][d];
            L += c * sm.l[w][g];
        }
        const int bh = b * a.Hq + h0 + g;
        if (a.n_splits == 1) {
            a.out[(size_t)bh * D + d] = L > 0.f ? acc / L : 0.f;
            if (d == 0 && a.lse) a.lse[bh] = L > 0.f ? (M + log2f(L)) * kEpLn2 : kEpNegInf;
        } else if (a.fused) {
            const size_t pi = (size_t)bh * a.n_splits + split;
            st_agent(a.part_o + pi * D + d, acc);
            if (d == 0) { st_agent(a.part_m + pi, M); st_agent(a.part_l + pi, L); }
        } else {
            const size_t pi = (size_t)bh * a.n_splits + split;
            a.part_o[pi * D + d] = acc;
            if (d == 0) { a.part_m[pi] = M; a.part_l[pi] = L; }
        }
    }
    if (a.n_splits == 1 || !a.fused) return;

    // Fused combine: every thread's coherent partial stores complete
    // (vmcnt 0), the barrier gathers the workgroup, one exchange counts the
    // arrival, and the workgroup that completes the group merges its splits.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long *cnt = a.counters + (size_t)b * a.Hkv * a.head_blocks + (size_t)kvh * a.head_blocks + hb;
        sm.last = arrive_last(cnt, a.epoch, active_splits(a, Tb)) ? 1 : 0;
    }
    __syncthreads();
    if (!sm.last) return;
    combine_group<WAVES, GB, D>(a, sm, b, h0, ng, active_splits(a, Tb));
}

}  // namespace fdk
