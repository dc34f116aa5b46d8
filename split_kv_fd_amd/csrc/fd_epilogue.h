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

// Count this workgroup's arrival at its group's counters and return true for
// the workgroup that completes the group (n_active arrivals).
//
// Each group has two 64-bit words holding (epoch << 32 | arrivals).  The
// first is counted with one fetch-add per workgroup: it is valid when it
// already carries this call's epoch, which the previous call on the same
// workspace leaves there (its last workgroup stores next_epoch << 32 with a
// zero count).  A word that carries anything else -- a new workspace,
// foreign data, a group the previous call did not finish -- sends every
// arrival of the call to the second word, counted with an exchange loop
// that restarts the count on a foreign epoch.  Within one call all arrivals
// see the same epoch in the first word (only the completing workgroup
// changes it, after every fetch-add), so they all take the same path.  The
// loop ends: every failed exchange means another workgroup's succeeded.
//
// The completing workgroup leaves both words in a state that depends on
// this call's arguments only: the first at (next_epoch << 32 | 0), the
// second at 0 (epoch 0, which no call uses).  A launch repeated with the
// same arguments -- a captured graph replayed, whose host passes
// epoch == next_epoch -- therefore counts from zero every time: through the
// fast word once the first replay has tagged it, through the cleared slow
// word before that.
//
// Ordering (LLVM AMDGPUUsage, memory model code sequences for GFX942, which
// gfx950 follows).  Every arriving workgroup publishes its partials with
// agent-scope atomic stores; all its threads wait for them (vmcnt 0) and
// meet at a barrier; then one thread issues an agent-scope release fence
// and counts the arrival with a relaxed RMW.  The workgroup whose RMW
// completes the group issues an agent-scope acquire fence: its RMW read a
// value in the release sequence every earlier arrival's RMW would head
// (all are RMWs on one word), so each earlier release fence synchronises
// with this acquire fence (the C++ fence rules, which the AMDGPU model
// follows), and the completing workgroup's other threads take that
// ordering over through a barrier before they load the partials (plain
// 16-byte loads: the writes happen before them, so they race with nothing;
// the acquire fence has also invalidated this compute unit's L1).  In the GFX942 sequences an agent-scope release
// fence is a write-back of the L2's dirty lines plus vmcnt(0), and an
// acquire fence vmcnt(0) plus an invalidate of the L2's non-local lines:
// one of each per arriving workgroup and per group (a stream-mode
// workgroup issues one release for all of its arrivals, at its end).
// FD_MERGE_RELEASE=0 builds the fence-free form (measurement only), which
// relies on the coherent sc1 stores and loads alone.
#ifndef FD_MERGE_RELEASE
#define FD_MERGE_RELEASE 1
#endif

__device__ __forceinline__ void release_fence() {
    if (FD_MERGE_RELEASE) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}

__device__ __forceinline__ bool arrive_last(unsigned long long *cnt, unsigned epoch, unsigned next_epoch,
                                            int n_active) {
    const unsigned long long old =
        __hip_atomic_fetch_add(cnt, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool last;
    if ((unsigned)(old >> 32) == epoch) {
        last = (unsigned)(old & 0xffffffffull) + 1u == (unsigned)n_active;
    } else {
        unsigned long long *slow = cnt + 1;
        unsigned long long prev = __hip_atomic_load(slow, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        unsigned long long next;
        for (;;) {
            next = ((unsigned)(prev >> 32) == epoch) ? prev + 1ull
                                                      : (((unsigned long long)epoch << 32) | 1ull);
            if (__hip_atomic_compare_exchange_strong(slow, &prev, next, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT))
                break;
        }
        last = (unsigned)(next & 0xffffffffull) == (unsigned)n_active;
    }
    if (last) {
        // every arrival of the group has counted: make their partials
        // visible here, then hand the words to the next call
        if (FD_MERGE_RELEASE) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(cnt + 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(cnt, (unsigned long long)next_epoch << 32, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    return last;
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

// Output row (index into out / lse rows) of query row r of kv head kvh of
// sequence b: query r / G, head kvh * G + r % G.
__device__ __forceinline__ size_t qrow(const SplitArgs &a, int b, int kvh, int r) {
    if (a.nq == 1) return (size_t)b * a.Hq + (size_t)kvh * a.G + r;
    const int i = r / a.G, g = r - i * a.G;
    return ((size_t)b * a.nq + i) * a.Hq + (size_t)kvh * a.G + g;
}

// A sequence with no tokens: out = 0 and lse = -inf for the block's rows.
// In fused mode no split of such a sequence reaches the merge, so split 0
// writes this instead.
template <int D>
__device__ void write_empty_group(const SplitArgs &a, int b, int kvh, int r0, int ng) {
    for (int idx = threadIdx.x; idx < ng * D; idx += blockDim.x) {
        const int g = idx / D, d = idx - (idx / D) * D;
        const size_t bh = qrow(a, b, kvh, r0 + g);
        a.out[bh * D + d] = 0.f;
        if (d == 0 && a.lse) a.lse[bh] = kEpNegInf;
    }
}

// Tokens of sequence b already in the cache (clamped to [0, T]).
__device__ __forceinline__ int cached_len(const SplitArgs &a, int b) {
    const int Tb = a.seq_lens ? a.seq_lens[b] : a.T;
    return Tb < 0 ? 0 : (Tb > a.T ? a.T : Tb);
}

// Tokens sequence b attends to: the cached ones, plus the new one when
// appending.
__device__ __forceinline__ int attended_len(const SplitArgs &a, int b) { return cached_len(a, b) + a.append; }

// Append: store the new token's key and value rows of (b, kvh) at token Tc
// of the cache -- row Tc of a contiguous cache when Tc < T, or row Tc % P of
// page page_table[b, Tc / P] when that column exists and names a pool page.
// Without such a slot nothing is stored (the token is still attended).  No
// workgroup of the launch reads that slot: every one that covers token Tc
// takes it from k_new / v_new.
template <int ROWB>
__device__ void store_new_token(const SplitArgs &a, int b, int kvh, int Tc) {
    size_t row;
    if (a.page_table) {
        const int col = Tc >> a.page_shift;
        const int page = col < a.max_pages ? a.page_table[(size_t)b * a.max_pages + col] : -1;
        if ((unsigned)page >= (unsigned)a.num_pages) return;
        row = ((size_t)page * a.Hkv + kvh) * (size_t)a.page_size + (size_t)(Tc & (a.page_size - 1));
    } else {
        if (Tc >= a.T) return;
        row = ((size_t)b * a.Hkv + kvh) * (size_t)a.T + (size_t)Tc;
    }
    const size_t src = ((size_t)b * a.Hkv + kvh) * (ROWB / 16);
    const uint4 *ks = static_cast<const uint4 *>(a.k_new) + src;
    const uint4 *vs = static_cast<const uint4 *>(a.v_new) + src;
    uint4 *kd = static_cast<uint4 *>(a.k_store) + row * (ROWB / 16);
    uint4 *vd = static_cast<uint4 *>(a.v_store) + row * (ROWB / 16);
    for (int i = threadIdx.x; i < ROWB / 16; i += blockDim.x) {
        kd[i] = ks[i];
        vd[i] = vs[i];
    }
}

// Splits that hold tokens of a sequence of length Tb.
__device__ __forceinline__ int active_splits(const SplitArgs &a, int Tb) {
    const int n = (Tb + a.chunk - 1) / a.chunk;
    return n < a.n_splits ? n : a.n_splits;
}

// Where one segment (a split, or a stream range of one row) leaves its
// result.  Partial row of head g for segment s: base + g*gs + s*ss.
struct SegOut {
    int final_out;                 // the segment is the whole row: write out / lse
    size_t base;
    int gs, ss, s;
    int fused;                     // the last arriving segment merges the group
    unsigned long long *cnt;       // the group's two arrival counter words
    int arrivals;                  // segments of the group (its merge count)
    int defer;                     // publish only: the caller counts the arrival later
    int ord;                       // stream mode: the segment's ordinal in its workgroup (clock marks)
};

__device__ __forceinline__ SegOut split_segment(const SplitArgs &a, int b, int kvh, int hb, int r0,
                                                int split, int Tb) {
    SegOut so;
    so.final_out = a.n_splits == 1;
    so.base = (((size_t)b * a.Hkv + kvh) * a.R + r0) * a.n_splits;
    so.gs = a.n_splits;
    so.ss = 1;
    so.s = split;
    so.fused = a.fused;
    so.cnt = a.counters + 2 * (((size_t)b * a.Hkv + kvh) * a.head_blocks + hb);
    so.arrivals = active_splits(a, Tb);
    so.defer = 0;
    so.ord = 3;
    return so;
}

// A partial's float4 in the merging workgroup.  With the release / acquire
// fences the partials are ordered before these reads (see arrive_last), so
// plain 16-byte loads serve; the fence-free measurement form keeps
// agent-scope atomic loads.
__device__ __forceinline__ float4 ld_part4(const float *p) {
    if (FD_MERGE_RELEASE) return *reinterpret_cast<const float4 *>(p);
    return make_float4(ld_agent(p), ld_agent(p + 1), ld_agent(p + 2), ld_agent(p + 3));
}

// Merge the last workgroup's group: for every valid head g of the block,
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the n active
// splits, read back from the workspace.  The loads of the split maxima and
// sums and of each thread's first PRE partial rows are issued together, and
// further splits are read PRE at a time, so a merge of n splits costs about
// n / (PRE*SG) memory round trips per pass.  Thread t owns
// one (head, float4 quad) pair and every SG-th split of it; sums run in
// split order within a thread and in split-group order across threads
// (deterministic).  ng * n <= kMergeMaxPairs.
template <int WAVES, int GB, int D>
__device__ void combine_group(const SplitArgs &a, EpilogueLds<WAVES, GB, D> &sm, const SegOut &so, int b,
                              int kvh, int r0, int ng, int n) {
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
            const size_t row = so.base + (size_t)g * so.gs + (size_t)s * so.ss;
            mr[k] = ld_agent(a.part_m + row);
            lr[k] = ld_agent(a.part_l + row);
        }
    }
    for (int p0 = 0; p0 < pairs; p0 += per_pass) {
        const int p = p0 + t / SG, sg = t - (t / SG) * SG;
        const bool active = p < pairs;
        const int g = active ? p / Q : 0, q = active ? p - (p / Q) * Q : 0;
        const size_t bh = qrow(a, b, kvh, r0 + g);
        const float *po = a.part_o + (so.base + (size_t)g * so.gs) * D + 4 * q;
        const size_t srow = (size_t)so.ss * D;
        float4 pre[PRE];
#pragma unroll
        for (int j = 0; j < PRE; ++j) {
            const int s = sg + j * SG;
            pre[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (active && s < n) pre[j] = ld_part4(po + (size_t)s * srow);
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
            // the rest, PRE splits per round trip (same order of sums)
            for (; s < n; s += PRE * SG) {
                float4 v[PRE];
#pragma unroll
                for (int j = 0; j < PRE; ++j) {
                    const int sj = s + j * SG;
                    v[j] = sj < n ? ld_part4(po + (size_t)sj * srow) : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int j = 0; j < PRE; ++j) {
                    const int sj = s + j * SG;
                    if (sj < n) {
                        const float c = wg[sj];
                        acc.x = fmaf(c, v[j].x, acc.x); acc.y = fmaf(c, v[j].y, acc.y);
                        acc.z = fmaf(c, v[j].z, acc.z); acc.w = fmaf(c, v[j].w, acc.w);
                    }
                }
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
            reinterpret_cast<float4 *>(a.out + bh * D)[q] = o;
            if (q == 0 && a.lse) a.lse[bh] = L > 0.f ? (sm.gm[g] + log2f(L)) * kEpLn2 : kEpNegInf;
        }
        __syncthreads();
    }
}

// Count a published segment's arrival and, in the workgroup that
// completes its group, merge the group.  Called by every thread; `fence`
// issues the release fence first (once per workgroup covers every arrival
// counted after it).
template <int WAVES, int GB, int D>
__device__ void arrive_and_merge(const SplitArgs &a, EpilogueLds<WAVES, GB, D> &sm, const SegOut &so, int b,
                                 int kvh, int r0, int ng, bool fence) {
    // every thread's coherent partial stores complete (vmcnt 0), the barrier
    // gathers the workgroup, one thread counts the arrival
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        if (fence) release_fence();
        sm.last = arrive_last(so.cnt, a.epoch, a.next_epoch, so.arrivals) ? 1 : 0;
    }
    __syncthreads();
    if (!sm.last) return;
    combine_group<WAVES, GB, D>(a, sm, so, b, kvh, r0, ng, so.arrivals);
}

// Called by every thread after sm.o / sm.m / sm.l hold each wave's state
// (the caller has synchronised).  Writes this segment's result and, in fused
// mode, completes the group when this workgroup arrives last (unless
// so.defer: then the caller counts the arrival later).
template <int WAVES, int GB, int D>
__device__ void finish_split(const SplitArgs &a, EpilogueLds<WAVES, GB, D> &sm, const SegOut &so, int b,
                             int kvh, int r0, int ng) {
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
        const size_t bh = qrow(a, b, kvh, r0 + g);
        const size_t pi = so.base + (size_t)g * so.gs + (size_t)so.s * so.ss;
        if (so.final_out) {
            a.out[bh * D + d] = L > 0.f ? acc / L : 0.f;
            if (d == 0 && a.lse) a.lse[bh] = L > 0.f ? (M + log2f(L)) * kEpLn2 : kEpNegInf;
        } else if (so.fused) {
            st_agent(a.part_o + pi * D + d, acc);
            if (d == 0) { st_agent(a.part_m + pi, M); st_agent(a.part_l + pi, L); }
        } else {
            a.part_o[pi * D + d] = acc;
            if (d == 0) { a.part_m[pi] = M; a.part_l[pi] = L; }
        }
    }
    if (so.final_out || !so.fused || so.defer) return;
    arrive_and_merge<WAVES, GB, D>(a, sm, so, b, kvh, r0, ng, true);
}

// Stream mode.  Rows (batch, kv head, head block) are padded to
// a.stream_align tokens, each row is preceded by a.stream_row_cost positions
// that hold no tokens, and the rows are laid end to end; workgroup w takes
// the stream range [w*per, (w+1)*per), which may cover the end of one row,
// whole rows and the start of another.  The positions before a row stand for
// the fixed time a segment costs (page staging, the latency of its first
// loads, the partial's write) in tokens' worth, so a range that holds more
// row starts gets fewer tokens.  Every workgroup scans the sequence lengths
// to find its range (B <= kStreamMaxB).  The segment of row r taken by
// workgroup w writes partial slot r + w (distinct for all rows and
// workgroups, and consecutive within a row); a row's last arriving segment
// merges it, and a row covered by one segment writes out directly.
// `seg(b, kvh, hb, c0, c1, so)` runs one segment (tokens [c0, c1) of the
// row; c0 == c1 for a range that only covers padding or the positions before
// the tokens).  A range cuts at most two rows (its first and its last);
// their segments only publish their partials, and after its last segment
// the workgroup counts both arrivals behind one release fence,
// `arrive(b, kvh, hb, so, fence)` merging a row it completes.  Sequences of
// length 0 have no segments: their outputs are written here.
template <int NT, int D, typename Seg, typename Arrive>
__device__ void drive_stream(const SplitArgs &a, long long *pref, int hpb, Seg &&seg, Arrive &&arrive) {
    FD_MARK(a, 0);
    const int t = threadIdx.x;
    const int RB = a.Hkv * a.head_blocks;             // rows per sequence
    const int align = a.stream_align;
    auto real_len = [&](int b) { return attended_len(a, b); };
    auto pad_len = [&](int b) { return (long long)((real_len(b) + align - 1) / align) * align; };
    // a row's length in the stream: its padded tokens after row_cost
    // positions that stand for the fixed cost of starting a segment
    const long long V = a.stream_row_cost;
    auto stride = [&](int b) { const long long lb = pad_len(b); return lb > 0 ? lb + V : 0; };

    // exclusive prefix over sequences of RB * row stride, and the longest row
    __shared__ long long s_scan[NT];
    __shared__ long long s_max[NT];
    long long carry = 0, lmax = 0;
    for (int c = 0; c < a.B; c += NT) {
        const int b = c + t;
        const long long v = b < a.B ? stride(b) : 0;
        lmax = v > lmax ? v : lmax;
        s_scan[t] = v * RB;
        __syncthreads();
        for (int off = 1; off < NT; off <<= 1) {
            const long long x = t >= off ? s_scan[t - off] : 0;
            __syncthreads();
            s_scan[t] += x;
            __syncthreads();
        }
        if (b < a.B) pref[b + 1] = carry + s_scan[t];
        carry += s_scan[NT - 1];
        __syncthreads();
    }
    s_max[t] = lmax;
    if (t == 0) pref[0] = 0;
    __syncthreads();
    for (int off = NT / 2; off > 0; off >>= 1) {
        if (t < off) s_max[t] = s_max[t] > s_max[t + off] ? s_max[t] : s_max[t + off];
        __syncthreads();
    }
    const long long total = pref[a.B];
    const long long longest = s_max[0];
    const int w = blockIdx.x, NW = gridDim.x;
    long long per = (total + NW - 1) / NW;
    // keep every row within merge_cap segments
    const long long min_per = (longest + a.merge_cap - 2) / (a.merge_cap - 1);
    per = per > min_per ? per : min_per;
    per = (per + align - 1) / align * align;
    if (per < align) per = align;

    // sequences of length 0: out = 0, lse = -inf for all their query rows
    for (int b = w; b < a.B; b += NW)
        if (real_len(b) == 0)
            for (int idx = t; idx < a.nq * a.Hq * D; idx += NT) {
                const int h = idx / D, d = idx - (idx / D) * D;
                const size_t row = (size_t)b * a.nq * a.Hq + h;
                a.out[row * D + d] = 0.f;
                if (d == 0 && a.lse) a.lse[row] = kEpNegInf;
            }

    const long long g0 = (long long)w * per;
    const long long g1 = g0 + per < total ? g0 + per : total;
    if (g0 >= g1) return;
    // the sequence holding stream position g0: the last b with pref[b] <= g0
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (pref[mid] <= g0) lo = mid; else hi = mid - 1;
    }
    FD_MARK(a, 1);
    // cut rows whose arrival is counted at the end (uniform across the workgroup)
    SegOut pend[2];
    int pb[2], pk[2], npend = 0, nseg = 0;
    bool done = false;
    for (int b = lo; b < a.B && pref[b] < g1 && !done; ++b) {
        const long long sb = stride(b);
        if (sb == 0) continue;
        const int Tb = real_len(b);
        long long k = g0 > pref[b] ? (g0 - pref[b]) / sb : 0;
        for (; k < RB; ++k) {
            const long long rs = pref[b] + k * sb;     // row start in the stream
            if (rs >= g1) { done = true; break; }
            // this range's part of the row, then of its tokens (which start
            // V positions in)
            const long long s0 = g0 > rs ? g0 - rs : 0;
            const long long s1 = g1 - rs < sb ? g1 - rs : sb;
            const long long c0 = s0 > V ? s0 - V : 0;
            const long long c1p = s1 > V ? s1 - V : 0;
            const int c1 = (int)(c1p < Tb ? c1p : Tb);
            const int r = b * RB + (int)k;
            const int kvh = (int)k / a.head_blocks, hb = (int)k - kvh * a.head_blocks;
            const long long wf = rs / per, wl = (rs + sb - 1) / per;
            SegOut so;
            so.final_out = wf == wl;
            so.base = (size_t)(r + wf) * hpb;
            so.gs = 1;
            so.ss = hpb;
            so.s = (int)(w - wf);
            so.fused = 1;
            so.cnt = a.counters + 2 * (size_t)r;
            so.arrivals = (int)(wl - wf + 1);
            so.defer = !so.final_out && npend < 2;
            so.ord = nseg < 3 ? nseg : 3;
            ++nseg;
            __syncthreads();                       // LDS of the previous segment is free
            FD_MARK(a, 2 + 4 * so.ord);
            seg(b, kvh, hb, (int)c0, c1 > (int)c0 ? c1 : (int)c0, so);
            FD_MARK(a, 5 + 4 * so.ord);
            if (so.defer) {
                pend[npend] = so;
                pb[npend] = b;
                pk[npend] = (int)k;
                ++npend;
            }
        }
    }
    FD_MARK(a, 14);
    for (int i = 0; i < npend; ++i) {
        const int kvh = pk[i] / a.head_blocks, hb = pk[i] - kvh * a.head_blocks;
        __syncthreads();                           // LDS of the previous segment or merge is free
        arrive(pb[i], kvh, hb, pend[i], i == 0);
    }
    FD_MARK(a, 15);
}

}  // namespace fdk
