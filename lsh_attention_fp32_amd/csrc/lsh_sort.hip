// lsh_sort.hip -- step 2: stable sort of each (batch, head, round) segment by
// (bucket, position).
//
// Method: twgreatdaily.com walkthrough, section "1 LSH Attention" (two-level
// sort: by bucket number, then by position inside the bucket); ai-scholar.tech
// summary, section "・LSH Attention" (sort per bucket before chunking).
//
// Positions arrive in increasing order, so a stable counting sort on the
// bucket alone yields the (bucket, position) order. Two kernels:
//   count   per 4096-element tile: bucket histogram in LDS (plain atomics)
//   scatter per tile: first the slot where each of its (tile, bucket) runs
//           starts -- the segment's bucket totals, scanned, plus the counts
//           of the earlier tiles -- then each wave ranks its 1024 elements in
//           order; lanes with equal buckets are grouped by a ballot match, so
//           ranks are exact and the LDS counter of a hot bucket is bumped once
//           per wave step (skewed buckets do not serialise on LDS atomics).
#include "lsh_internal.h"

namespace lsh {

size_t sort_workspace_bytes(const Dims& d) {
    return align_up(sizeof(int32_t) * (size_t)d.segs * d.nb * (size_t)sort_ntiles(d), 256);
}

// Mask of the lanes whose bucket equals this lane's (0 for inactive lanes).
__device__ __forceinline__ uint64_t match_bucket(int b, int nbits, bool active) {
    uint64_t m = __ballot(active);
    for (int k = 0; k < nbits; ++k) {
        const bool bit = (b >> k) & 1;
        const uint64_t s = __ballot(active && bit);
        m &= bit ? s : ~s;
    }
    return active ? m : 0ull;
}

// Bucket ids outside [0, nb) are a caller error; clamping keeps every LDS
// access in bounds (the result is then unspecified, never a fault).
__device__ __forceinline__ int clamp_bucket(int b, int nb) {
    return (int)min((unsigned)b, (unsigned)(nb - 1));
}

__device__ __forceinline__ uint64_t lanes_below_s(int lane) {
    return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// counts layout: [seg][tile][bucket] (each tile writes one contiguous row)
__global__ __launch_bounds__(256) void sort_count_kernel(const int32_t* __restrict__ buckets,
                                                         Dims dm, int ntiles,
                                                         int32_t* __restrict__ counts) {
    extern __shared__ int32_t hist[];
    const int tile = blockIdx.x;
    const int64_t seg = blockIdx.y;
    for (int b = threadIdx.x; b < dm.nb; b += 256) hist[b] = 0;
    __syncthreads();
    const int32_t* src = buckets + seg * dm.L;
    const int64_t beg = (int64_t)tile * kSortTile;
    const int64_t end = min(beg + (int64_t)kSortTile, (int64_t)dm.L);
    // A count needs no order: plain LDS atomics (lanes of one instruction that
    // hit the same bucket serialise, which only a heavily skewed tile feels).
    constexpr int PER = kSortTile / 256;
    int b[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int64_t i = beg + k * 256 + threadIdx.x;
        b[k] = i < end ? clamp_bucket(src[i], dm.nb) : -1;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k)
        if (b[k] >= 0) atomicAdd(&hist[b[k]], 1);
    __syncthreads();
    for (int b = threadIdx.x; b < dm.nb; b += 256)
        counts[(seg * ntiles + tile) * dm.nb + b] = hist[b];
}

constexpr int kScatterXcds = 8;   // L2 domains of the chip

// PACKED: perm[slot] = (bucket << kPackPosBits) | position and no inverse.
template <bool PACKED>
__global__ __launch_bounds__(256) void sort_scatter_kernel(const int32_t* __restrict__ buckets,
                                                           const int32_t* __restrict__ offs,
                                                           Dims dm, int ntiles, int nbits,
                                                           int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ inv) {
    extern __shared__ int32_t sh[];   // [kSortWaves][nb] counts, then running slots; [nb] run starts
    __shared__ int32_t wsum[4];
    constexpr int SUB = kSortTile / kSortWaves;
    // Workgroups are dealt round-robin over the L2 domains (id % kScatterXcds):
    // every tile of a segment gets the same residue, so one L2 collects the
    // segment's scattered 4-byte writes and hands whole lines to memory.
    const int64_t id = blockIdx.x, k = id / kScatterXcds;
    const int64_t seg = (k / ntiles) * kScatterXcds + id % kScatterXcds;
    const int tile = (int)(k % ntiles);
    if (seg >= dm.segs) return;   // the grid is rounded up to whole domain groups
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nb = dm.nb;
    int32_t* start = sh + kSortWaves * nb;

    // The wave's 1024 bucket ids are loaded first (all in flight while the
    // run starts are computed) and stay in registers.
    const int32_t* src = buckets + seg * dm.L;
    const int64_t wbeg = (int64_t)tile * kSortTile + (int64_t)wave * SUB;
    const int64_t wend = min(wbeg + (int64_t)SUB, (int64_t)dm.L);
    constexpr int STEPS = SUB / kWave;
    int kb[STEPS], rank[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int64_t i = wbeg + s * kWave + lane;
        kb[s] = i < wend ? clamp_bucket(src[i], nb) : 0;
    }

    // First slot of this tile's run of every bucket: exclusive scan over
    // buckets of the segment totals, plus the counts of the earlier tiles.
    // Totals (start[]) and earlier-tile counts (sh[0..nb)) are gathered with
    // coalesced reads, then scanned in contiguous chunks of bpt buckets.
    {
        const int32_t* cnt = offs + seg * ntiles * nb;
        for (int b = threadIdx.x; b < nb; b += 256) {
            int32_t tot = 0, before = 0;
#pragma unroll 16
            for (int t = 0; t < ntiles; ++t) {
                const int32_t c = cnt[(int64_t)t * nb + b];
                tot += c;
                before += t < tile ? c : 0;
            }
            start[b] = tot;
            sh[b] = before;
        }
        __syncthreads();
        const int bpt = (nb + 255) / 256;
        const int b0 = threadIdx.x * bpt;
        int32_t mine = 0;
        for (int j = 0; j < bpt; ++j)
            if (b0 + j < nb) mine += start[b0 + j];
        int32_t incl = mine;
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t o = __shfl_up(incl, off);
            if (lane >= off) incl += o;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int32_t run = incl - mine;
        for (int w = 0; w < wave; ++w) run += wsum[w];
        for (int j = 0; j < bpt; ++j)
            if (b0 + j < nb) {
                const int32_t tot = start[b0 + j];
                start[b0 + j] = run + sh[b0 + j];
                run += tot;
            }
    }
    __syncthreads();
    for (int k = threadIdx.x; k < kSortWaves * nb; k += 256) sh[k] = 0;
    __syncthreads();
    int32_t* mine = sh + wave * nb;
    // Pass 1 ranks every element among the wave's earlier elements of its
    // bucket (ballot match, so exact and stable) while counting; pass 2 only
    // adds the (wave, bucket) run start and stores.
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const bool active = wbeg + s * kWave + lane < wend;
        const uint64_t m = match_bucket(kb[s], nbits, active);
        rank[s] = mine[kb[s]] + __popcll(m & lanes_below_s(lane));
        // every lane has read its bucket's count; leaders now advance them
        __builtin_amdgcn_wave_barrier();
        if (active && (__ffsll((long long)m) - 1) == lane) mine[kb[s]] += __popcll(m);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    // first slot of each (wave, bucket) run
    for (int b = threadIdx.x; b < nb; b += 256) {
        int32_t run = start[b];
        for (int w = 0; w < kSortWaves; ++w) {
            const int32_t c = sh[w * nb + b];
            sh[w * nb + b] = run;
            run += c;
        }
    }
    __syncthreads();
    // pass 2: slots
    int32_t* P = perm + seg * dm.L;
    int32_t* I = PACKED ? nullptr : inv + seg * dm.L;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int64_t i = wbeg + s * kWave + lane;
        if (i < wend) {
            const int32_t slot = mine[kb[s]] + rank[s];
            if constexpr (PACKED) {
                P[slot] = (int32_t)(((uint32_t)kb[s] << kPackPosBits) | (uint32_t)i);
            } else {
                P[slot] = (int32_t)i;
                I[i] = slot;
            }
        }
    }
}

hipError_t launch_sort(const int32_t* buckets, const Dims& d, int32_t* perm, int32_t* inv,
                       void* ws, hipStream_t st, hipEvent_t* ev, int* nev, const char** names,
                       bool packed) {
    const int ntiles = (int)sort_ntiles(d);
    int nbits = 0;
    while ((1 << nbits) < d.nb) ++nbits;
    int32_t* counts = (int32_t*)ws;
    dim3 grid((unsigned)ntiles, (unsigned)d.segs);
    hipError_t e;
    sort_count_kernel<<<grid, 256, sizeof(int32_t) * d.nb, st>>>(buckets, d, ntiles, counts);
    if ((e = mark(st, ev, nev, names, "sort_count")) != hipSuccess) return e;
    const size_t lds = sizeof(int32_t) * (kSortWaves + 1) * d.nb;
    const int64_t sgroups = (d.segs + kScatterXcds - 1) / kScatterXcds;
    const unsigned sgrid = (unsigned)(sgroups * kScatterXcds * ntiles);
    if (packed)
        sort_scatter_kernel<true><<<sgrid, 256, lds, st>>>(buckets, counts, d, ntiles, nbits,
                                                           perm, nullptr);
    else
        sort_scatter_kernel<false><<<sgrid, 256, lds, st>>>(buckets, counts, d, ntiles, nbits,
                                                            perm, inv);
    return mark(st, ev, nev, names, "sort_scatter");
}

}  // namespace lsh
