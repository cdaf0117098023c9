// lsh_sort.hip -- step 2: stable sort of each (batch, head, round) segment by
// (bucket, position).
//
// Method: twgreatdaily.com walkthrough, section "1 LSH Attention" (two-level
// sort: by bucket number, then by position inside the bucket); ai-scholar.tech
// summary, section "・LSH Attention" (sort per bucket before chunking).
//
// Positions arrive in increasing order, so a stable counting sort on the
// bucket alone yields the (bucket, position) order. Three kernels:
//   count   per 4096-element tile: bucket histogram in LDS (plain atomics),
//           written to counts[seg][tile][bucket]
//   prefix  per (segment, 256 buckets): each bucket's counts become the
//           number of that bucket in the segment's earlier tiles (in place),
//           and its total goes to totals[seg][bucket]
//   scatter per tile: the slot where each of its (tile, bucket) runs starts
//           is the exclusive scan of the segment's totals plus the tile's
//           prefix -- 2 nb values read per tile, whatever the number of
//           tiles -- then each of its 4, 8 or 16 waves ranks its share of
//           the tile in order; lanes with equal buckets are grouped by a
//           ballot match, so ranks are exact and the LDS counter of a hot
//           bucket is bumped once per wave step (skewed buckets do not
//           serialise on LDS atomics).
// A segment of one tile (L <= 4096) is its own tile: the tile-local order the
// scatter builds is the segment's order, so the count and prefix launches are
// skipped and the scatter alone sorts it. A segment of two to four tiles
// counts and prefixes in one launch (sort_count_prefix_kernel), and many
// segments of at most 1024 positions are sorted one per wave
// (sort_wave_kernel).
#include <mutex>

#include "lsh_internal.h"

namespace lsh {

// Static scratch of lsh_sort_noalloc: the sort's counts, prefixes and totals
// for callers that cannot allocate. Each GPU the library runs on holds its own
// copy until the process ends. In host code `scratch` names a host-side
// stand-in, never the device memory: only the address hipGetSymbolAddress
// returns (sort_scratch below) may reach a kernel or a copy.
static __device__ __align__(256) int32_t scratch[kSortScratchBytes / sizeof(int32_t)];

hipError_t sort_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        // once per device, with that device current
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

size_t sort_workspace_bytes(const Dims& d) {
    // counts (then earlier-tile prefixes) [seg][tile][nb], totals [seg][nb]
    return align_up(sizeof(int32_t) * (size_t)d.segs * d.nb * (size_t)sort_ntiles(d), 256) +
           align_up(sizeof(int32_t) * (size_t)d.segs * d.nb, 256);
}

// Mask of the lanes whose bucket equals this lane's (0 for inactive lanes).
// For bit k, the ballot s of the lanes with the bit set, xor'ed with this
// lane's bit spread over a word (0 or all ones), is the set of lanes that
// differ from it in bit k; the lanes that differ in no bit match.
__device__ __forceinline__ uint64_t match_bucket(int b, int nbits, bool active) {
    uint32_t miss_lo = 0, miss_hi = 0;
    for (int k = 0; k < nbits; ++k) {
        const int32_t spread = __builtin_amdgcn_sbfe((int32_t)b, k, 1);   // 0 or -1
        const uint64_t s = __ballot(spread != 0);
        miss_lo |= (uint32_t)s ^ (uint32_t)spread;
        miss_hi |= (uint32_t)(s >> 32) ^ (uint32_t)spread;
    }
    const uint64_t m = __ballot(active) & ~(((uint64_t)miss_hi << 32) | miss_lo);
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
    const int64_t seg = block_y();
    if (seg >= dm.segs) return;
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

// A segment of at most kCPTiles tiles (and kCPBuckets buckets) counts and
// prefixes in one workgroup of 1024 threads, so neither the per-tile counts
// nor a second launch go through global memory first: every element adds
// one to its tile's row of an LDS histogram [tile][bucket] (plain LDS
// atomics, as in sort_count_kernel), then one thread per bucket walks the
// tiles and writes the earlier-tile counts and the segment total, the same
// outputs as sort_count_kernel followed by sort_prefix_kernel. Longer
// segments keep the two launches, which spread a segment over one workgroup
// per tile: at 16K positions the fused kernel takes 11 us against 16 us for
// the pair, at 64K 29 us against 18 us (64 segments fill 64 compute units).
constexpr int kCPThreads = 1024;
constexpr int kCPTiles = 4;
constexpr int kCPBuckets = 2048;

__global__ __launch_bounds__(kCPThreads) void sort_count_prefix_kernel(
    const int32_t* __restrict__ buckets, Dims dm, int ntiles, int32_t* __restrict__ counts,
    int32_t* __restrict__ totals) {
    extern __shared__ int32_t hist[];   // [ntiles][nb]
    const int64_t seg = block_y();
    if (seg >= dm.segs) return;
    const int nb = dm.nb, L = dm.L;
    for (int i = threadIdx.x; i < ntiles * nb; i += kCPThreads) hist[i] = 0;
    __syncthreads();
    const int32_t* src = buckets + seg * L;
    constexpr int U = 8;   // loads in flight per thread
    for (int i0 = 0; i0 < L; i0 += U * kCPThreads) {
        int b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * kCPThreads + threadIdx.x;
            b[u] = i < L ? clamp_bucket(src[i], nb) : -1;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * kCPThreads + threadIdx.x;
            if (b[u] >= 0) atomicAdd(&hist[(i / kSortTile) * nb + b[u]], 1);
        }
    }
    __syncthreads();
    for (int b = threadIdx.x; b < nb; b += kCPThreads) {
        int32_t run = 0;
        for (int t = 0; t < ntiles; ++t) {
            const int32_t c = hist[t * nb + b];
            counts[(seg * ntiles + t) * nb + b] = run;
            run += c;
        }
        totals[seg * nb + b] = run;
    }
}

// counts[seg][t][b] -> number of b in tiles 0 .. t-1 of the segment (in
// place); totals[seg][b] = number of b in the segment. One thread per bucket,
// so every tile's row is read and written with coalesced accesses; the loads
// of kBatch tiles are issued before any is used.
__global__ __launch_bounds__(256) void sort_prefix_kernel(int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ totals, int nb,
                                                          int ntiles, int64_t segs) {
    constexpr int kBatch = 8;
    const int b = blockIdx.x * 256 + threadIdx.x;
    const int64_t seg = block_y();
    if (b >= nb || seg >= segs) return;
    int32_t* c = counts + seg * ntiles * nb + b;
    int32_t run = 0;
    for (int t0 = 0; t0 < ntiles; t0 += kBatch) {
        int32_t x[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) x[k] = t0 + k < ntiles ? c[(int64_t)(t0 + k) * nb] : 0;
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
            if (t0 + k < ntiles) {
                c[(int64_t)(t0 + k) * nb] = run;
                run += x[k];
            }
    }
    totals[seg * nb + b] = run;
}

constexpr int kScatterXcds = 8;   // L2 domains of the chip

// Exclusive scan of a[0..n) in LDS by the T threads of the workgroup (each
// takes a contiguous chunk, then a wave scan and the earlier waves' sums).
// Ends with a barrier; a[] is read and written only between barriers.
template <int T>
__device__ __forceinline__ void block_exclusive_scan(int32_t* a, int n, int32_t* wsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int per = (n + T - 1) / T;
    const int b0 = threadIdx.x * per;
    int32_t mine = 0;
    for (int j = 0; j < per; ++j)
        if (b0 + j < n) mine += a[b0 + j];
    int32_t incl = mine;
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int32_t run = incl - mine;
    for (int w = 0; w < wave; ++w) run += wsum[w];
    for (int j = 0; j < per; ++j)
        if (b0 + j < n) {
            const int32_t c = a[b0 + j];
            a[b0 + j] = run;
            run += c;
        }
    __syncthreads();
}

// PACKED: perm[slot] = (bucket << kPackPosBits) | position and no inverse.
// STAGED (positions below 2^kPackPosBits): the tile's elements are first put
// in their sorted order in LDS, then written out with consecutive threads on
// consecutive slots, so each (tile, bucket) run leaves as one contiguous
// piece instead of one 4-byte store per element at scattered slots.
// W waves per workgroup share a tile, each ranking a contiguous 1/W of it.
template <bool PACKED, bool STAGED, bool ONE_TILE, int W>
__global__ __launch_bounds__(64 * W) void sort_scatter_kernel(const int32_t* __restrict__ buckets,
                                                           const int32_t* __restrict__ prefix,
                                                           const int32_t* __restrict__ totals,
                                                           Dims dm, int ntiles, int nbits,
                                                           int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ inv) {
    constexpr int T = 64 * W;
    // LDS: [W][nb] per-wave counts, then run starts; [nb] the tile's
    // first slot of each bucket (later: slot minus tile-local index); STAGED:
    // [kSortTile] the tile's keys in sorted order, whose first nb entries
    // hold the tile-local bucket starts before the keys are written
    extern __shared__ int32_t sh[];
    __shared__ int32_t wsum[W];
    static_assert(!PACKED || STAGED, "packed keys are staged");
    static_assert(!ONE_TILE || STAGED, "a one-tile segment is sorted in its staged order");
    constexpr int SUB = kSortTile / W;
    // Workgroups are dealt round-robin over the L2 domains (id % kScatterXcds):
    // every tile of a segment gets the same residue, so one L2 collects the
    // segment's writes and hands whole lines to memory.
    const int64_t id = blockIdx.x, k = id / kScatterXcds;
    const int64_t seg = (k / ntiles) * kScatterXcds + id % kScatterXcds;
    const int tile = (int)(k % ntiles);
    if (seg >= dm.segs) return;   // the grid is rounded up to whole domain groups
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nb = dm.nb;
    int32_t* start = sh + W * nb;
    int32_t* lkeys = start + nb;

    // The wave's bucket ids (at most SUB) are loaded first (all in flight while the
    // run starts are computed) and stay in registers.
    const int32_t* src = buckets + seg * dm.L;
    const int64_t tbeg = (int64_t)tile * kSortTile;
    // a one-tile segment shorter than the tile spreads over all W waves
    // (whole 64-element steps each), so each wave's ranking chain is 1/W of
    // the segment instead of one wave doing up to SUB elements
    const int sub = ONE_TILE ? (int)min((int64_t)SUB, (dm.L + T - 1) / T * kWave) : SUB;
    const int64_t wbeg = tbeg + (int64_t)wave * sub;
    const int64_t wend = min(wbeg + (int64_t)sub, (int64_t)dm.L);
    constexpr int STEPS = SUB / kWave;
    int kb[STEPS], rank[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int64_t i = wbeg + s * kWave + lane;
        kb[s] = i < wend ? clamp_bucket(src[i], nb) : 0;
    }

    // First slot of this tile's run of every bucket: exclusive scan over
    // buckets of the segment totals, plus this bucket's count in the earlier
    // tiles (both read with coalesced loads). A one-tile segment needs
    // neither: its slots are the tile-local ones.
    if constexpr (!ONE_TILE) {
        const int32_t* tot = totals + seg * nb;
        const int32_t* pre = prefix + (seg * ntiles + tile) * nb;
        for (int b = threadIdx.x; b < nb; b += T) {
            start[b] = tot[b];
            sh[b] = pre[b];
        }
        __syncthreads();
        block_exclusive_scan<T>(start, nb, wsum);
        for (int b = threadIdx.x; b < nb; b += T) start[b] += sh[b];
    }
    __syncthreads();
    for (int k = threadIdx.x; k < W * nb; k += T) sh[k] = 0;
    __syncthreads();
    int32_t* mine = sh + wave * nb;
    // Pass 1 ranks every element among the wave's earlier elements of its
    // bucket (ballot match, so exact and stable) while counting; pass 2 only
    // adds the (wave, bucket) run start and stores.
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        if (wbeg + s * kWave >= wend) break;   // wave-uniform
        const bool active = wbeg + s * kWave + lane < wend;
        const uint64_t m = match_bucket(kb[s], nbits, active);
        rank[s] = mine[kb[s]] + __popcll(m & lanes_below_s(lane));
        // every lane has read its bucket's count; leaders now advance them
        __builtin_amdgcn_wave_barrier();
        if (active && (__ffsll((long long)m) - 1) == lane) mine[kb[s]] += __popcll(m);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    if constexpr (STAGED) {
        // tile-local start of every bucket (scan of the tile's counts), then
        // each (wave, bucket) run's local start; start[] becomes slot - local
        int32_t* lstart = lkeys;
        for (int b = threadIdx.x; b < nb; b += T) {
            int32_t c = 0;
            for (int w = 0; w < W; ++w) c += sh[w * nb + b];
            lstart[b] = c;
        }
        __syncthreads();
        block_exclusive_scan<T>(lstart, nb, wsum);
        for (int b = threadIdx.x; b < nb; b += T) {
            int32_t run = lstart[b];
            start[b] = ONE_TILE ? 0 : start[b] - run;
            for (int w = 0; w < W; ++w) {
                const int32_t c = sh[w * nb + b];
                sh[w * nb + b] = run;
                run += c;
            }
        }
        __syncthreads();   // lstart is dead from here on: its space takes the keys
        int32_t* I = PACKED ? nullptr : inv + seg * dm.L;
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const int64_t i = wbeg + s * kWave + lane;
            if (i < wend) {
                const int32_t local = mine[kb[s]] + rank[s];
                lkeys[local] = (int32_t)(((uint32_t)kb[s] << kPackPosBits) | (uint32_t)i);
                if constexpr (!PACKED) I[i] = local + start[kb[s]];
            }
        }
        __syncthreads();
        int32_t* P = perm + seg * dm.L;
        const int n = (int)min((int64_t)kSortTile, (int64_t)dm.L - tbeg);
        for (int i = threadIdx.x; i < n; i += T) {
            const uint32_t key = (uint32_t)lkeys[i];
            const int32_t slot = i + start[key >> kPackPosBits];
            P[slot] = PACKED ? (int32_t)key : (int32_t)(key & kPackPosMask);
        }
    } else {
        // first slot of each (wave, bucket) run
        for (int b = threadIdx.x; b < nb; b += T) {
            int32_t run = start[b];
            for (int w = 0; w < W; ++w) {
                const int32_t c = sh[w * nb + b];
                sh[w * nb + b] = run;
                run += c;
            }
        }
        __syncthreads();
        // pass 2: every element straight to its slot
        int32_t* P = perm + seg * dm.L;
        int32_t* I = inv + seg * dm.L;
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const int64_t i = wbeg + s * kWave + lane;
            if (i < wend) {
                const int32_t slot = mine[kb[s]] + rank[s];
                P[slot] = (int32_t)i;
                I[i] = slot;
            }
        }
    }
}

// A segment of at most kWaveSeg positions (and at most kWaveSegBuckets
// buckets) is sorted by one wave on its own, four segments per workgroup and
// no workgroup barrier: the wave ranks its elements with the ballot match of
// the scatter, keeping the bucket counts in its own LDS slice; one wave-wide
// exclusive scan over the buckets turns the counts into run starts; each
// element's key goes to its slot in a wave-private LDS staging row, which is
// then written out in slot order. (Through the one-tile scatter such a
// segment kept one of the workgroup's four waves busy.) Used when there are
// more than kWaveSortSegs segments; fewer go to the one-tile scatter, whose
// four waves split a segment so each ranking chain is a quarter as long (at
// 64 x 1K positions the sort takes 9.7 against 16.2 us with one round, 16.4
// against 17.9 with four, 23.4 against 20.7 with eight).
constexpr int kWaveSeg = kSortTile / kSortWaves;   // 1024
constexpr int kWaveSegBuckets = 1024;
constexpr int64_t kWaveSortSegs = 2048;   // eight segments per compute unit

template <bool PACKED>
__global__ __launch_bounds__(256) void sort_wave_kernel(const int32_t* __restrict__ buckets,
                                                        Dims dm, int nbits,
                                                        int32_t* __restrict__ perm,
                                                        int32_t* __restrict__ inv) {
    extern __shared__ int32_t sh[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t seg = (int64_t)blockIdx.x * kSortWaves + wave;
    if (seg >= dm.segs) return;   // the whole wave leaves; no workgroup barrier follows
    const int nb = dm.nb, L = dm.L;
    int32_t* cnt = sh + wave * (kWaveSegBuckets + kWaveSeg);
    int32_t* lkeys = cnt + kWaveSegBuckets;
    const int32_t* src = buckets + seg * L;
    constexpr int STEPS = kWaveSeg / kWave;
    int kb[STEPS], rank[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int i = s * kWave + lane;
        kb[s] = i < L ? clamp_bucket(src[i], nb) : 0;
    }
    for (int b = lane; b < nb; b += kWave) cnt[b] = 0;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        if (s * kWave >= L) break;   // wave-uniform
        const bool active = s * kWave + lane < L;
        const uint64_t m = match_bucket(kb[s], nbits, active);
        rank[s] = cnt[kb[s]] + __popcll(m & lanes_below_s(lane));
        __builtin_amdgcn_wave_barrier();
        if (active && (__ffsll((long long)m) - 1) == lane) cnt[kb[s]] += __popcll(m);
        __builtin_amdgcn_wave_barrier();
    }
    // counts -> run starts: each lane takes a contiguous run of buckets
    const int per = (nb + kWave - 1) / kWave;
    const int b0 = lane * per;
    int32_t mine = 0;
    for (int j = 0; j < per; ++j)
        if (b0 + j < nb) mine += cnt[b0 + j];
    int32_t incl = mine;
    for (int off = 1; off < kWave; off <<= 1) {
        const int32_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    int32_t run = incl - mine;
    __builtin_amdgcn_wave_barrier();
    for (int j = 0; j < per; ++j)
        if (b0 + j < nb) {
            const int32_t c = cnt[b0 + j];
            cnt[b0 + j] = run;
            run += c;
        }
    __builtin_amdgcn_wave_barrier();
    int32_t* I = PACKED ? nullptr : inv + seg * L;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int i = s * kWave + lane;
        if (i < L) {
            const int32_t slot = cnt[kb[s]] + rank[s];
            lkeys[slot] = (int32_t)(((uint32_t)kb[s] << kPackPosBits) | (uint32_t)i);
            if constexpr (!PACKED) I[i] = slot;
        }
    }
    __builtin_amdgcn_wave_barrier();
    int32_t* P = perm + seg * L;
    for (int i = lane; i < L; i += kWave) {
        const uint32_t key = (uint32_t)lkeys[i];
        P[i] = PACKED ? (int32_t)key : (int32_t)(key & kPackPosMask);
    }
}

// Waves per scatter workgroup: more waves shorten each wave's ranking chain
// (a tile's elements are split among them) at the cost of W per-wave count
// rows of nb entries to clear, scan and walk, and of fewer workgroups per
// compute unit. Chosen from same-box measurements of the scatter (4 / 8 / 16
// waves): 16 x 4K positions, 128 buckets, one round 19.0 / 13.1 / 10.9 us,
// eight rounds 23.7 / 20.7 / 23.3; 8 x 8 x 4K, 64 buckets 19.2 / 13.7 / 11.3;
// 64 x 1K, 32 buckets 10.0 / 8.8 / 9.4; four-tile segments at 4 x 16K, 512
// buckets 18.6 / 13.2 (8 waves); 16-tile segments at 64K, 1024 buckets
// 29.7 / 32.1 (8 waves); 16-tile segments at 64K, 2048 buckets (whole sort)
// 43.9 / 35.5 us on 128 workgroups, 44.8 / 37.2 on 256, 48.9 / 53.1 on 512.
static int scatter_waves(const Dims& d, bool one) {
    const int64_t wgs = d.segs * sort_ntiles(d);
    if (one && d.L >= 2048 && d.nb <= 512 && wgs <= 4096) return 16;
    if (d.nb <= 512 || (one && d.nb <= 1024) || (wgs <= 256 && d.nb <= 2048)) return 8;
    return 4;
}

hipError_t launch_sort(const int32_t* buckets, const Dims& d, int32_t* perm, int32_t* inv,
                       void* ws, hipStream_t st, hipEvent_t* ev, int* nev, const char** names,
                       bool packed) {
    const int ntiles = (int)sort_ntiles(d);
    int nbits = 0;
    while ((1 << nbits) < d.nb) ++nbits;
    int32_t* counts = (int32_t*)ws;
    int32_t* totals =
        (int32_t*)((char*)ws + align_up(sizeof(int32_t) * (size_t)d.segs * d.nb * ntiles, 256));
    const dim3 grid = grid_split((unsigned)ntiles, d.segs);
    hipError_t e;
    // staged needs positions below 2^kPackPosBits (a packed key per element)
    const bool staged = packed_sort_keys(d);
    if (packed && !staged) return hipErrorInvalidValue;
    const bool one = staged && ntiles == 1;
    if (staged && d.L <= kWaveSeg && d.nb <= kWaveSegBuckets && d.segs > kWaveSortSegs) {
        static_assert(kWaveSeg <= (1 << kPackPosBits), "wave segments use packed keys");
        const unsigned wgrid = (unsigned)((d.segs + kSortWaves - 1) / kSortWaves);
        const size_t wlds = sizeof(int32_t) * kSortWaves * (kWaveSegBuckets + kWaveSeg);
        if (packed)
            sort_wave_kernel<true><<<wgrid, 256, wlds, st>>>(buckets, d, nbits, perm, nullptr);
        else
            sort_wave_kernel<false><<<wgrid, 256, wlds, st>>>(buckets, d, nbits, perm, inv);
        return mark(st, ev, nev, names, "sort_scatter");
    }
    if (!one && ntiles <= kCPTiles && d.nb <= kCPBuckets) {
        sort_count_prefix_kernel<<<grid_split(1, d.segs), kCPThreads,
                                   sizeof(int32_t) * ntiles * d.nb, st>>>(buckets, d, ntiles,
                                                                          counts, totals);
        if ((e = mark(st, ev, nev, names, "sort_count")) != hipSuccess) return e;
    } else if (!one) {
        sort_count_kernel<<<grid, 256, sizeof(int32_t) * d.nb, st>>>(buckets, d, ntiles, counts);
        if ((e = mark(st, ev, nev, names, "sort_count")) != hipSuccess) return e;
        sort_prefix_kernel<<<grid_split((unsigned)((d.nb + 255) / 256), d.segs), 256, 0, st>>>(
            counts, totals, d.nb, ntiles, d.segs);
        if ((e = mark(st, ev, nev, names, "sort_prefix")) != hipSuccess) return e;
    }
    static_assert(kSortTile >= kMaxBuckets, "the staged keys' space first holds nb starts");
    const int64_t sgroups = (d.segs + kScatterXcds - 1) / kScatterXcds;
    const unsigned sgrid = (unsigned)(sgroups * kScatterXcds * ntiles);
    const int W = scatter_waves(d, one);
#define LSH_SCATTER(P, S, O, INV, WW)                                                          \
    sort_scatter_kernel<P, S, O, WW>                                                           \
        <<<sgrid, 64 * WW, sizeof(int32_t) * ((WW + 1) * d.nb + (S ? kSortTile : 0)), st>>>( \
            buckets, counts, totals, d, ntiles, nbits, perm, INV)
#define LSH_SCATTER_W(P, S, O, INV)          \
    do {                                     \
        if (W == 16)                         \
            LSH_SCATTER(P, S, O, INV, 16);   \
        else if (W == 8)                     \
            LSH_SCATTER(P, S, O, INV, 8);    \
        else                                 \
            LSH_SCATTER(P, S, O, INV, 4);    \
    } while (0)
    if (packed && one)
        LSH_SCATTER_W(true, true, true, nullptr);
    else if (packed)
        LSH_SCATTER_W(true, true, false, nullptr);
    else if (one)
        LSH_SCATTER_W(false, true, true, inv);
    else if (staged)
        LSH_SCATTER_W(false, true, false, inv);
    else
        LSH_SCATTER(false, false, false, inv, 4);
#undef LSH_SCATTER_W
#undef LSH_SCATTER
    return mark(st, ev, nev, names, "sort_scatter");
}

}  // namespace lsh
