// moe_permute: stable counting sort of the T*k (token, expert) pairs by expert.
//
// Gathering each expert's rows into one contiguous block, with an offset array
// marking where each group starts, is the layout the grouped GEMM needs
// ("从 Dense GEMM 到 TP MoE 的演进逻辑", sections 2.1 and 2.2).
//
// Up to kOneMaxPairs pairs (512 tokens x top-8, 4096 x top-2) one workgroup
// of 1024 threads does all of it in LDS, in one launch: wave w owns the w-th
// sixteenth of the pairs; every thread reads the ids coalesced, keeps each
// clamped id as a byte in LDS and counts it in its owner wave's histogram
// (LDS atomics); threads 0..E-1 turn the histograms into each wave's first
// row per expert (wavefront shuffle scan over experts); each wave then
// scatters its own pairs in order as below, so the result is the same stable
// sort.  Its time is launch and memory latency plus ~1 ns per pair (one CU
// issues every scattered index store), so larger inputs, where three launches
// spread over many CUs cost less, use three small kernels over fixed chunks
// of kChunk consecutive pairs:
//   count    per-chunk histogram of expert ids (LDS counters)
//   scan     per expert, exclusive scan of its chunk counts -> the base row of
//            each (chunk, expert); exclusive scan over experts (wavefront
//            shuffle scans, then the four wavefront totals) -> offsets
//   scatter  one wavefront per chunk walks its pairs in order, 64 at a time;
//            lanes holding the same expert find each other with one ballot per
//            id bit, take rank = #peers on lower lanes, and the highest peer
//            advances that expert's running base.  Pair order is kept, so the
//            result equals a stable sort: bit-exact and deterministic.
#include "common.h"

namespace moe {
namespace {

constexpr int kChunk = 1024;
constexpr int kOneWaves = 16;            // waves of the one-workgroup permute
constexpr int kOneMaxPairs = 8192;       // its largest input (512 pairs per wave)

__device__ __forceinline__ int clamp_id(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

__global__ __launch_bounds__(256) void permute_count_kernel(const int32_t* __restrict__ ids,
                                                            int P, int E,
                                                            int32_t* __restrict__ counts)
{
    __shared__ int hist[MOE_MAX_EXPERTS];
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    const int p0 = blockIdx.x * kChunk;
    const int p1 = min(P, p0 + kChunk);
    for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x) atomicAdd(&hist[clamp_id(ids[p], E)], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// One block of 256 threads: thread e owns expert e (E <= 256).
__global__ __launch_bounds__(256) void permute_scan_kernel(int32_t* __restrict__ counts,
                                                           int nchunks, int T, int P, int E,
                                                           int n_shared,
                                                           int32_t* __restrict__ offsets)
{
    constexpr int kBatch = 16;  // loads in flight per thread (the column walk is latency bound)
    __shared__ int wtot[4];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        // pass 1: this expert's total over all chunks
        for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
            int v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                v[j] = (c0 + j < nchunks) ? counts[(size_t)(c0 + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < kBatch; ++j) run += v[j];
        }
    }
    // exclusive scan over experts: an inclusive scan within each wavefront
    // (six shuffle steps), then the four wavefront totals through LDS
    const int lane = e & 63, wave = e >> 6;
    int incl = (e < E) ? run : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
    }
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wtot[w];
    const int base = (e < E) ? before + incl - run : 0;
    if (e < E) {
        offsets[e] = base;
        // pass 2: each chunk's count becomes its first row for this expert
        int acc = base;
        for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
            int v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                v[j] = (c0 + j < nchunks) ? counts[(size_t)(c0 + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (c0 + j < nchunks) counts[(size_t)(c0 + j) * E + e] = acc;
                acc += v[j];
            }
        }
    }
    if (e == 0) {
        offsets[E] = P;
        for (int s = 0; s < n_shared; ++s) offsets[E + s + 1] = P + (s + 1) * T;
    }
}

// Rank the 64 pairs [pb, pb + 64) of a wave (those below p1) among equal
// expert ids, in lane order: rows run[e] + rank, run[e] advanced by the
// group's size.  One ballot per id bit finds each lane's peers.
// `e` is this lane's (clamped) expert id, ignored past p1.
__device__ __forceinline__ void scatter_step(int pb, int p1, int e, int nbits, int P, int lane,
                                             uint64_t lower, int* run,
                                             int32_t* __restrict__ permuted_pair,
                                             int32_t* __restrict__ unpermute)
{
    const int p = pb + lane;
    const bool valid = p < p1;
    if (!valid) e = 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = __ballot(valid && bit);
        peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lower);
    const int r0 = valid ? run[e] : 0;
    // every lane has read run[] before the highest peer of a group advances it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (valid) {
        const int row = r0 + rank;
        if (row < P) {  // always true when the counts match the ids
            permuted_pair[row] = p;
            unpermute[p] = row;
        }
        if ((peers >> lane) == 1ull)  // highest lane of its peer group
            run[e] = r0 + __popcll(peers);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One wavefront per chunk.
__global__ __launch_bounds__(64) void permute_scatter_kernel(const int32_t* __restrict__ ids,
                                                             int P, int E,
                                                             const int32_t* __restrict__ base,
                                                             int32_t* __restrict__ permuted_pair,
                                                             int32_t* __restrict__ unpermute)
{
    __shared__ int run[MOE_MAX_EXPERTS];
    const int lane = threadIdx.x;
    for (int e = lane; e < E; e += 64) run[e] = base[(size_t)blockIdx.x * E + e];
    __syncthreads();
    const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
    const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int p0 = blockIdx.x * kChunk;
    const int p1 = min(P, p0 + kChunk);
    // the chunk's ids, all loads in flight at once (one memory latency per
    // chunk instead of one per 64 pairs)
    constexpr int kIter = kChunk / 64;
    static_assert(kChunk % 64 == 0, "whole waves per chunk");
    int idv[kIter];
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
        const int p = p0 + it * 64 + lane;
        idv[it] = p < p1 ? ids[p] : 0;
    }
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
        if (p0 + it * 64 >= p1) break;  // past the last pair (wave-uniform)
        scatter_step(p0 + it * 64, p1, clamp_id(idv[it], E), nbits, P, lane, lower, run, permuted_pair,
                     unpermute);
    }
}

__global__ __launch_bounds__(kOneWaves * 64) void permute_one_kernel(const int32_t* __restrict__ ids,
                                                                     int P, int T, int E, int n_shared,
                                                                     int32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ permuted_pair,
                                                                     int32_t* __restrict__ unpermute)
{
    constexpr int kThreads = kOneWaves * 64;
    constexpr int kBatch = kOneMaxPairs / kThreads;  // every ids load in flight at once
    __shared__ int cnt[kOneWaves][MOE_MAX_EXPERTS];  // per wave: counts, then running rows
    __shared__ uint8_t sid[kOneMaxPairs];            // clamped expert id of every pair (E <= 256)
    __shared__ int wtot[4];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar loops below
    for (int i = tid; i < kOneWaves * MOE_MAX_EXPERTS; i += kThreads) (&cnt[0][0])[i] = 0;
    __syncthreads();
    // wave w owns pairs [p0, p1): whole groups of 64 except at the end; every
    // p < P has owner p / per < kOneWaves
    const int per = ((P + kOneWaves - 1) / kOneWaves + 63) & ~63;
    const int p0 = min(P, wave * per), p1 = min(P, p0 + per);
    // every thread reads ids coalesced, kBatch loads in flight, keeps the
    // clamped id in LDS and counts it for the pair's owner wave
    for (int b0 = 0; b0 < P; b0 += kBatch * kThreads) {
        int v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int p = b0 + j * kThreads + tid;
            v[j] = p < P ? ids[p] : 0;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int p = b0 + j * kThreads + tid;
            if (p < P) {
                const int e = clamp_id(v[j], E);
                sid[p] = (uint8_t)e;
                atomicAdd(&cnt[p / per][e], 1);
            }
        }
    }
    __syncthreads();
    // thread e < E (waves 0..3): expert total, exclusive scan over experts
    int tot = 0, incl = 0;
    if (tid < MOE_MAX_EXPERTS) {
        if (tid < E)
            for (int w = 0; w < kOneWaves; ++w) tot += cnt[w][tid];
        incl = tot;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        if (lane == 63) wtot[wave] = incl;
    }
    __syncthreads();
    if (tid < E) {
        int base = incl - tot;
        for (int w = 0; w < wave; ++w) base += wtot[w];
        offsets[tid] = base;
        // each wave's first row for this expert: after every earlier wave's pairs
        for (int w = 0; w < kOneWaves; ++w) {
            const int c = cnt[w][tid];
            cnt[w][tid] = base;
            base += c;
        }
    }
    if (tid == 0) {
        offsets[E] = P;
        for (int sh = 0; sh < n_shared; ++sh) offsets[E + sh + 1] = P + (sh + 1) * T;
    }
    __syncthreads();
    const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
    const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int pb = p0; pb < p1; pb += 64) {  // wave-uniform
        const int p = pb + lane;
        scatter_step(pb, p1, p < p1 ? (int)sid[p] : 0, nbits, P, lane, lower, cnt[wave], permuted_pair,
                     unpermute);
    }
}

}  // namespace

size_t permute_scratch_bytes(int T, int k, int E)
{
    const size_t P = (size_t)T * k;
    const size_t nchunks = (P + kChunk - 1) / kChunk;
    return nchunks * (size_t)E * sizeof(int32_t);
}

moe_status launch_permute(const int32_t* ids, int T, int k, int E, int n_shared,
                          int32_t* offsets, int32_t* permuted_pair, int32_t* unpermute,
                          void* ws, hipStream_t s)
{
    const int P = T * k;
    if (P <= kOneMaxPairs) {
        {
            TimedLaunch tl(MOE_KID_PERMUTE_ONE, s);
            hipLaunchKernelGGL(permute_one_kernel, dim3(1), dim3(kOneWaves * 64), 0, s, ids, P, T, E,
                               n_shared, offsets, permuted_pair, unpermute);
        }
        return launch_status("permute_one_kernel");
    }
    const int nchunks = (P + kChunk - 1) / kChunk;
    int32_t* counts = static_cast<int32_t*>(ws);
    {
        TimedLaunch tl(MOE_KID_PERMUTE_COUNT, s);
        hipLaunchKernelGGL(permute_count_kernel, dim3(nchunks), dim3(256), 0, s, ids, P, E,
                           counts);
    }
    moe_status st = launch_status("permute_count_kernel");
    if (st != MOE_OK) return st;
    {
        TimedLaunch tl(MOE_KID_PERMUTE_SCAN, s);
        hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(256), 0, s, counts, nchunks, T, P,
                           E, n_shared, offsets);
    }
    st = launch_status("permute_scan_kernel");
    if (st != MOE_OK) return st;
    {
        TimedLaunch tl(MOE_KID_PERMUTE_SCATTER, s);
        hipLaunchKernelGGL(permute_scatter_kernel, dim3(nchunks), dim3(64), 0, s, ids, P, E,
                           counts, permuted_pair, unpermute);
    }
    return launch_status("permute_scatter_kernel");
}

}  // namespace moe
