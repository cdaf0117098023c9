// lsh_hash.hip -- step 1: angular LSH, bucket = first argmax of [x R_r, -x R_r].
//
// Method: ultralytics.com glossary "Reformer", section "Atenção LSH" (random
// matrix R of shape [rounds, d, n_buckets/2], bucket = index of the largest
// entry of [xR, -xR]); twgreatdaily.com walkthrough, section "1 LSH Attention"
// (one hash function per round, rounds independent).
//
// The argmax over [p, -p] is the column with the largest |p|, on the "-" half
// when that p is negative; exact ties resolve to the lowest index of the
// concatenation.
//
// Design (gfx950):
//  * Fast pass on the matrix cores in fp16. Each round's R is scaled by the
//    power of two that brings its largest |R| into [2^14, 2^15) and rounded to
//    fp16 (R_s); each token's x (bf16: at most 8 significant bits) is scaled
//    the same way by its own power of two (x_s), which makes the conversion
//    exact except for elements more than 2^28 below the token's largest.
//    Scaling a row or a whole round changes no argmax. fp16 products are exact
//    in fp32 and the MFMA accumulates in fp32. Each lane keeps the three
//    largest |p| of its token as packed keys (|p| with the low mantissa bits
//    replaced by (column << 1 | sign)), three integer min/max operations per
//    value.
//  * Certification. Every fast value is within
//        E = |x_s| (rho_r + c |R_s|max) + sqrt(d) 2^-14 |R_s|max
//    of the exact scaled projection: rho_r bounds |R_s,b - fp16(R_s,b)| (the
//    prep pass computes it from the actual roundings, Cauchy-Schwarz does the
//    rest), c bounds the fp32 accumulation, and the last term covers x
//    elements a matrix core may flush as fp16 subnormals. If the top key beats
//    the second by more than 2E (plus the key quantisation), the bucket is the
//    exact argmax. If only the third is certainly out, the token-round is
//    queued with its two candidate columns; otherwise with a request to scan
//    every column.
//  * Re-decision in fp64 on the GPU for the queued token-rounds (a few
//    percent for Gaussian x and R).
//  * fp32 inputs (or head sizes without a matrix-core kernel) use a plain fp32
//    FMA pass with the same certification and re-decision.
#include <algorithm>

#include "lsh_internal.h"

namespace lsh {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

static constexpr float kTwoM24 = 5.9604644775390625e-8f;   // 2^-24

// ------------------------------------------------------------------ workspace
static size_t rfrag_elems(const Dims& d) {
    // [nr][ntiles][d/16 k-steps][64 lanes][8] fp16
    return (size_t)d.nr * hash_ntiles(d) * kHashColTile * d.d;
}

static size_t rt_elems(const Dims& d) {
    // [nr][ntiles * 32 columns][d] float32
    return (size_t)d.nr * hash_ntiles(d) * kHashColTile * d.d;
}

size_t hash_workspace_bytes(const Dims& d) {
    size_t b = 256;                                              // counter
    b += align_up(sizeof(float) * 3 * d.nr * hash_ntiles(d), 256);   // tnorm
    b += align_up(sizeof(uint16_t) * rfrag_elems(d), 256);       // rfrag
    b += align_up(sizeof(float) * rt_elems(d), 256);             // rt
    b += align_up(sizeof(RefineItem) * (size_t)queue_tokens(d) * d.nh, 256);   // queue
    b += align_up(sizeof(int32_t) * 2 * (size_t)queue_tokens(d) / kWave * d.nh, 256);   // rcount
    b += align_up(sizeof(int32_t) * d.nr, 256);                                          // scount
    b += align_up(sizeof(int32_t) * (size_t)queue_tokens(d) * d.nr, 256);                // slist
    b += align_up(sizeof(uint64_t) * (size_t)queue_tokens(d) * d.nr, 256);               // sbest
    return b;
}

HashWorkspace carve_hash_workspace(void* ws, const Dims& d) {
    char* p = (char*)ws;
    HashWorkspace w;
    w.counter = (int32_t*)p;
    w.vmax = (uint32_t*)(p + 3 * sizeof(int32_t));
    p += 256;
    w.tnorm = (float*)p;
    p += align_up(sizeof(float) * 3 * d.nr * hash_ntiles(d), 256);
    w.rfrag = (uint16_t*)p;
    p += align_up(sizeof(uint16_t) * rfrag_elems(d), 256);
    w.rt = (float*)p;
    p += align_up(sizeof(float) * rt_elems(d), 256);
    w.queue = (RefineItem*)p;
    p += align_up(sizeof(RefineItem) * (size_t)queue_tokens(d) * d.nh, 256);
    w.rcount = (int32_t*)p;
    p += align_up(sizeof(int32_t) * 2 * (size_t)queue_tokens(d) / kWave * d.nh, 256);
    w.scount = (int32_t*)p;
    p += align_up(sizeof(int32_t) * d.nr, 256);
    w.slist = (int32_t*)p;
    p += align_up(sizeof(int32_t) * (size_t)queue_tokens(d) * d.nr, 256);
    w.sbest = (uint64_t*)p;
    return w;
}

// ------------------------------------------------------------------ R prep
// One workgroup per (round, 32-column tile) of R, staged through LDS:
//  * e_r from max|R| of the round: a round of one tile (n_buckets <= 64,
//    ONE) takes it from the tile it stages; otherwise every workgroup of the
//    round reads the whole round (L2 hits after the first), so all agree on
//    the scale without a launch of its own;
//  * tnorm[bound][round][tile]: the tile's largest column 2-norm of R, of
//    R_s and of the residual (sums of squares in fp32, then rounded up),
//    stored without atomics; readers take the maximum over the round's tiles;
//  * rt    = R transposed to [round][column][k] in fp32 (padded columns are 0),
//            read by the fp64 re-decision;
//  * rfrag = fp16(R * 2^e_r) in the A-operand order of
//            v_mfma_f32_32x32x16_f16: for (round, tile, k-step), 64 lanes of 8
//            values, lane l holding column tile*32 + l%32 and
//            k = kstep*16 + 8*(l/32) + e.
// Workgroup (0, 0) also clears the re-decision count, max|v| and the
// per-round list counts, which later passes fill in.
template <bool ONE>
__global__ __launch_bounds__(256) void rprep_kernel(const float* __restrict__ R, int d, int half,
                                                    int ntiles, int nh,
                                                    float* __restrict__ tnorm,
                                                    float* __restrict__ rt,
                                                    uint16_t* __restrict__ rfrag,
                                                    int32_t* __restrict__ counter,
                                                    int32_t* __restrict__ scount) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    __shared__ float tile[128][kHashColTile + 1];
    __shared__ float wmax[4];
    const int t = blockIdx.x;
    const int r = (int)block_y();   // R round, of nh
    if (r >= nh) return;
    if (t == 0 && r == 0) {
        if (threadIdx.x < 4) counter[threadIdx.x] = 0;
        for (int i = threadIdx.x; i < nh; i += 256) scount[i] = 0;
    }
    const float* Rr = R + (int64_t)r * d * half;
    const int col0 = t * kHashColTile;
    float m = 0.f;
#pragma unroll 8
    for (int idx = threadIdx.x; idx < d * kHashColTile; idx += 256) {
        const int k = idx / kHashColTile, c = idx % kHashColTile;
        const float a = (col0 + c < half) ? Rr[(int64_t)k * half + col0 + c] : 0.f;
        tile[k][c] = a;
        m = fmaxf(m, fabsf(a));
    }
    // max |R| of the round: from this tile when it is the round, else from the
    // whole round (a contiguous d * half floats, 16-byte aligned as R and d
    // are), read the same way by every workgroup of the round
    if constexpr (!ONE) {
        m = 0.f;
        const f32x4* R4 = (const f32x4*)Rr;
        const int n4 = d * half / 4;
#pragma unroll 8
        for (int i = threadIdx.x; i < n4; i += 256) {
            const f32x4 q = R4[i];
            m = fmaxf(m, fmaxf(fmaxf(fabsf(q[0]), fabsf(q[1])), fmaxf(fabsf(q[2]), fabsf(q[3]))));
        }
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const int e = 15 - __builtin_amdgcn_frexp_expf(M);   // M * 2^e in [2^14, 2^15)

    {   // 8 threads per column, d/8 rows each
        const int c = threadIdx.x >> 3, part = threadIdx.x & 7, klen = d / 8;
        float s0 = 0.f, s1 = 0.f, s2 = 0.f;
        for (int k = part * klen; k < (part + 1) * klen; ++k) {
            const float a = tile[k][c];
            const float as = ldexpf(a, e);
            const float res = as - (float)(_Float16)as;   // exact
            s0 = fmaf(a, a, s0);
            s1 = fmaf(as, as, s1);
            s2 = fmaf(res, res, s2);
        }
        for (int off = 1; off < 8; off <<= 1) {
            s0 += __shfl_xor(s0, off);
            s1 += __shfl_xor(s1, off);
            s2 += __shfl_xor(s2, off);
        }
        // fp32 sums of d squares: relative error below d * 2^-24; sqrt halves it
        const float up = 1.0f + (float)(d + 4) * kTwoM24;
        const float flush = sqrtf((float)d) * 1.0001f * 6.103515625e-05f;   // sqrt(d) 2^-14
        const bool real = col0 + c < half;
        float n0 = real ? sqrtf(s0) * up : 0.f;
        float n1 = real ? sqrtf(s1) * up : 0.f;
        float n2 = real ? sqrtf(s2) * up + flush : 0.f;
        // the tile's largest, then one atomic max per workgroup and bound
        for (int off = 8; off < 64; off <<= 1) {
            n0 = fmaxf(n0, __shfl_xor(n0, off));
            n1 = fmaxf(n1, __shfl_xor(n1, off));
            n2 = fmaxf(n2, __shfl_xor(n2, off));
        }
        __shared__ float wn[3][4];
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        if (lane == 0) {
            wn[0][wave] = n0;
            wn[1][wave] = n1;
            wn[2][wave] = n2;
        }
        __syncthreads();
        if (threadIdx.x < 3)
            tnorm[((int64_t)threadIdx.x * nh + r) * ntiles + t] =
                fmaxf(fmaxf(wn[threadIdx.x][0], wn[threadIdx.x][1]),
                      fmaxf(wn[threadIdx.x][2], wn[threadIdx.x][3]));
    }
    float* dst = rt + ((int64_t)r * ntiles * kHashColTile + col0) * d;
    for (int idx = threadIdx.x; idx < d * kHashColTile; idx += 256) {
        const int c = idx / d, k = idx % d;
        dst[idx] = tile[k][c];
    }
    const int ks = d / 16;
    for (int f = threadIdx.x; f < ks * kWave; f += 256) {
        const int l = f & 63, s = f >> 6;
        const int c = l & 31, k0 = s * 16 + 8 * (l >> 5);
        uint32_t w[4];
        for (int e2 = 0; e2 < 4; ++e2) {
            const _Float16 h0 = (_Float16)ldexpf(tile[k0 + 2 * e2][c], e);
            const _Float16 h1 = (_Float16)ldexpf(tile[k0 + 2 * e2 + 1][c], e);
            w[e2] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        }
        u32x4 pk = {w[0], w[1], w[2], w[3]};
        *(u32x4*)(rfrag + (((int64_t)r * ntiles + t) * ks * kWave + f) * 8) = pk;
    }
}

// ------------------------------------------------------------------ helpers
// Keys are non-negative floats (bit 31 clear, never NaN for finite inputs), so
// float ordering equals the ordering of their bit patterns. With k1 >= k2 >= k3,
// inserting a key is two medians and a max.
__device__ __forceinline__ void top3_insert(float& k1, float& k2, float& k3, float key) {
    k3 = __builtin_amdgcn_fmed3f(k2, key, k3);
    k2 = __builtin_amdgcn_fmed3f(k1, key, k2);
    k1 = __uint_as_float(max(__float_as_uint(k1), __float_as_uint(key)));
}

__device__ __forceinline__ uint64_t lanes_below(int lane) {
    return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// A wave's appends to its own queue region (see RefineItem): ballots give
// each flagged lane its place; the running counts stay wave-uniform.
struct RegionWriter {
    RefineItem* base;   // the region's first item
    int size;           // items in the region
    int n0, n1;         // two-candidate items (front), full scans (back)

    __device__ __forceinline__ void push(bool flag, const RefineItem& it, int lane) {
        const uint64_t any = __ballot(flag);
        if (!any) return;
        const uint64_t m1 = __ballot(flag && it.mode == 1);
        const uint64_t m0 = any & ~m1;
        if (flag) {
            if (it.mode == 1)
                base[size - 1 - (n1 + __popcll(m1 & lanes_below(lane)))] = it;
            else
                base[n0 + __popcll(m0 & lanes_below(lane))] = it;
        }
        n0 += __popcll(m0);
        n1 += __popcll(m1);
    }
    __device__ __forceinline__ void finish(int32_t* rcount, int64_t region, int lane) const {
        if (lane == 0) {
            rcount[2 * region] = n0;
            rcount[2 * region + 1] = n1;
        }
    }
};

// Decision shared by both fast passes. v1 >= v2 >= v3 are the three largest
// fast |p| values (as floats), thr the certification threshold.
__device__ __forceinline__ int classify(float v1, float v2, float v3, float thr) {
    if (v1 - v2 > thr) return -1;  // certified
    if (v1 - v3 > thr) return 0;   // two candidates
    return 1;                      // scan every column
}

// ------------------------------------------------------------------ re-decision, part 1
// Run by each wave of a fast pass on its own queue region when its sweep is
// done (it wrote the region itself, so no other wave is involved): the
// two-candidate items are decided in fp64 from the fp32 transpose of R, 16 at
// a time, 4 lanes per item (lane l4 takes elements 16 j + 4 l4 + e, so the
// four lanes of an item read 64 contiguous bytes per load), the next items
// fetched a pass ahead. Full-scan items are moved to their round's list for
// the grouped scan (a per-round atomic ticket; such items are rare). The exact
// rule: largest |p| = |x . R_b| over [p, -p], ties to the lowest index of the
// concatenation (a p of either zero sign counts as "+").
template <typename T>
__device__ __forceinline__ void refine_region(const T* __restrict__ qk,
                                              const float* __restrict__ rt, const Dims& dm,
                                              const RefineItem* rq, int region_size, int n0,
                                              int n1, int lane, int32_t* __restrict__ buckets,
                                              int32_t* __restrict__ scount,
                                              int32_t* __restrict__ slist,
                                              uint64_t* __restrict__ sbest, int64_t cap) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const int half = dm.nb / 2;
    const int hpad = ((half + kHashColTile - 1) / kHashColTile) * kHashColTile;
    const int D = dm.d;
    const int sub = lane >> 2, l4 = lane & 3, ksteps = D / 16;
    // the region's entries were stored by this wave's lanes: make them visible
    // to the other lanes before reading them back
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    RefineItem nxt = sub < n0 ? rq[sub] : RefineItem{0, -1, -1, 0};
    for (int q0 = 0; q0 < n0; q0 += 16) {
        const bool ok = q0 + sub < n0;
        const RefineItem it = nxt;
        if (q0 + 16 + sub < n0) nxt = rq[q0 + 16 + sub];   // next pass's item, in flight
        const bool va = it.a >= 0 && it.a < half, vb = it.b >= 0 && it.b < half && it.b != it.a;
        double pa = 0.0, pb = 0.0;
        if (ok) {
            const int i = it.item % dm.L, rest = it.item / dm.L;
            const int r = rest % dm.nh, bh = rest / dm.nh;
            const T* x = qk + ((int64_t)bh * dm.L + i) * D + 4 * l4;
            const float* Rr = rt + (int64_t)r_round(dm, bh, r) * hpad * D;   // [column][k]
            const float* ra = Rr + (int64_t)(va ? it.a : 0) * D + 4 * l4;
            const float* rb = Rr + (int64_t)(vb ? it.b : 0) * D + 4 * l4;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j < ksteps) {
                    const f32x4 A = *(const f32x4*)(ra + 16 * j);
                    const f32x4 B = *(const f32x4*)(rb + 16 * j);
                    const f32x4 X = IO<T>::load4(x, 16 * j);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pa += (double)X[e] * (double)A[e];
                        pb += (double)X[e] * (double)B[e];
                    }
                }
        }
        for (int off = 2; off > 0; off >>= 1) {
            pa += __shfl_xor(pa, off);
            pb += __shfl_xor(pb, off);
        }
        if (ok && l4 == 0) {
            const int ca = it.a + (pa < 0.0 ? half : 0), cb = it.b + (pb < 0.0 ? half : 0);
            int pick;
            if (!vb) pick = ca;
            else if (!va) pick = cb;
            else if (fabs(pa) > fabs(pb)) pick = ca;
            else if (fabs(pb) > fabs(pa)) pick = cb;
            else pick = min(ca, cb);
            buckets[it.item] = pick;
        }
    }
    for (int q = lane; q < n1; q += kWave) {
        const int32_t item = rq[region_size - 1 - q].item;
        const int rest = item / dm.L;
        const int r = r_round(dm, rest / dm.nh, rest % dm.nh);   // lists are per R round
        const int slot = atomicAdd(&scount[r], 1);
        slist[(int64_t)r * cap + slot] = item;
        sbest[(int64_t)r * cap + slot] = 0ull;
    }
}

// ------------------------------------------------------------------ fast pass (MFMA)
// One workgroup = 4 waves; a wave owns 32*TOKF tokens (TOKF B-operand
// fragments kept in registers for the whole kernel) and sweeps every column
// tile of every round; R tiles stream through LDS, double-buffered.
//
// When `v` is given, the kernel also folds max|v| over its tokens' value rows
// into *vmax (as a bf16 bit pattern; one atomic max per workgroup): the scale
// of the fp16 per-round outputs of the fused forward comes for the price of a
// read that overlaps the matrix-core work.
template <int D, int TOKF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void hash_mfma_kernel(const uint16_t* __restrict__ qk,
                                                        const u32x4* __restrict__ rfrag,
                                                        const float* __restrict__ tnorm, Dims dm,
                                                        int32_t* __restrict__ buckets,
                                                        RefineItem* __restrict__ queue,
                                                        int32_t* __restrict__ rcount,
                                                        const uint16_t* __restrict__ v,
                                                        uint32_t* __restrict__ vmax,
                                                        const float* __restrict__ rt,
                                                        int32_t* __restrict__ scount,
                                                        int32_t* __restrict__ slist,
                                                        uint64_t* __restrict__ sbest,
                                                        int64_t cap) {
    constexpr int KS = D / 16;
    constexpr int TILE_U4 = KS * kWave;         // 16-byte lane fragments per column tile
    constexpr int PRE = TILE_U4 / 256;          // fragments each thread stages
    constexpr int TOK_WAVE = 32 * TOKF;
    constexpr int TOK_WG = 4 * TOK_WAVE;
    constexpr float kAcc = (float)(4 * D + 8) * kTwoM24;          // fp32 accumulation
    constexpr float kFlushX = (D == 64 ? 8.0001f : 11.3138f) * 6.103515625e-05f;   // sqrt(d) 2^-14
    __shared__ u32x4 lds[2][TILE_U4];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = dm.nb / 2;
    const int ntiles = (half + kHashColTile - 1) / kHashColTile;
    const int total = dm.nh * ntiles;
    // The workgroup's tokens: TOK_WG consecutive token-heads. With per-head
    // rotations they stay inside one (batch, head), whose R rounds start at vr0.
    int64_t wg_first = (int64_t)blockIdx.x * TOK_WG, wg_end = dm.T;
    int vr0 = 0;
    if (dm.per_head_r) {
        const int nblk = (dm.L + TOK_WG - 1) / TOK_WG;
        const int64_t bh = blockIdx.x / nblk;
        wg_first = bh * dm.L + (int64_t)(blockIdx.x - bh * nblk) * TOK_WG;
        wg_end = (bh + 1) * dm.L;
        vr0 = r_round(dm, bh, 0);
    }
    const int64_t tok0 = wg_first + (int64_t)wave * TOK_WAVE;
    const u32x4* rf = rfrag + (int64_t)vr0 * ntiles * TILE_U4;   // this head's R tiles
    // this wave's queue region: its tokens, every round
    const int64_t region = (int64_t)blockIdx.x * 4 + wave;
    RegionWriter qw{queue + region * TOK_WAVE * dm.nh, TOK_WAVE * dm.nh, 0, 0};
    // key = |p| with its low `bits` mantissa bits replaced by the column
    const int bits = 32 - __clz(ntiles * kHashColTile - 1);
    const uint32_t keymask = 0x7FFFFFFFu & ~((1u << bits) - 1u);
    const float qerr = __uint_as_float((uint32_t)(127 + bits - 22) << 23) + 9.5367431640625e-7f;

    // B operand: lane holds x_s[tok0 + f*32 + lane%32][16 s + 8 (lane/32) + e]
    // in fp16, x_s = x * 2^e with the token's largest |x| brought into [2^14, 2^15).
    // The raw rows and (when asked) this workgroup's value rows are all
    // requested before any of them is used, so their latencies overlap.
    u32x4 ux[TOKF][KS];
#pragma unroll
    for (int f = 0; f < TOKF; ++f) {
        const int64_t tok = tok0 + f * 32 + (lane & 31);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            ux[f][s] = (u32x4){0u, 0u, 0u, 0u};
            if (tok < wg_end) ux[f][s] = ((const u32x4*)(qk + tok * D))[2 * s + (lane >> 5)];
        }
    }
    __shared__ uint32_t wvmax[4];
    if (v) {
        // this workgroup's tokens are one contiguous run of value rows
        constexpr int NV = TOK_WG * (D / 8) / 256;   // 16-byte pieces per thread
        const int64_t first = wg_first;
        const int64_t nvec = min((int64_t)TOK_WG, wg_end - first) * (D / 8);
        const u32x4* src = (const u32x4*)(v + first * D);
        u32x4 vw[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int64_t i = threadIdx.x + 256 * j;
            vw[j] = i < nvec ? src[i] : (u32x4){0u, 0u, 0u, 0u};
        }
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) m = max(m, max(vw[j][e] & 0x7FFFu, (vw[j][e] >> 16) & 0x7FFFu));
        for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
        if (lane == 0) wvmax[wave] = m;
    }
    f16x8 xb[TOKF][KS];
    float xn2[TOKF];
#pragma unroll
    for (int f = 0; f < TOKF; ++f) {
        uint32_t mb = 0;   // largest |x| as bf16 bits (integer order = float order)
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e) mb = max(mb, max(ux[f][s][e] & 0x7FFFu, (ux[f][s][e] >> 16) & 0x7FFFu));
        mb = max(mb, (uint32_t)__shfl_xor((int)mb, 32));
        const int xe = 15 - __builtin_amdgcn_frexp_expf(__uint_as_float(mb << 16));
        xn2[f] = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 h;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = ldexpf(__uint_as_float(ux[f][s][e] << 16), xe);
                const float b = ldexpf(__uint_as_float(ux[f][s][e] & 0xFFFF0000u), xe);
                xn2[f] = fmaf(a, a, fmaf(b, b, xn2[f]));
                h[e] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
                       ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
            }
            xb[f][s] = __builtin_bit_cast(f16x8, h);
        }
        xn2[f] += __shfl_xor(xn2[f], 32);
    }
    // flat index of (token, round 0) in buckets [B,H,nh,L]; round r adds r*L
    int32_t item0[TOKF];
    bool tok_live[TOKF];
#pragma unroll
    for (int f = 0; f < TOKF; ++f) {
        const int64_t tok = tok0 + f * 32 + (lane & 31);
        tok_live[f] = tok < wg_end;
        const int64_t bh = tok / dm.L, i = tok - bh * dm.L;
        item0[f] = tok_live[f] ? (int32_t)(bh * dm.nh * dm.L + i) : 0;
    }

    for (int i = threadIdx.x; i < TILE_U4; i += 256) lds[0][i] = rf[i];
    // each round's two certification bounds (R_s norm, residual norm): the
    // largest over the round's column tiles, once per workgroup, in LDS
    // (dynamic: 2 * n_hashes floats)
    extern __shared__ float rbound[];
    for (int i = threadIdx.x; i < 2 * dm.nh; i += 256) {
        const int b = 1 + i / dm.nh, rr = vr0 + i % dm.nh;
        const float* tb = tnorm + ((int64_t)b * dm.nr + rr) * ntiles;
        float m = 0.f;
        for (int j = 0; j < ntiles; ++j) m = fmaxf(m, tb[j]);
        rbound[i] = m;
    }
    __syncthreads();
    if (v && threadIdx.x == 0)
        atomicMax(vmax, max(max(wvmax[0], wvmax[1]), max(wvmax[2], wvmax[3])));

    float k1[TOKF], k2[TOKF], k3[TOKF];
    // the round's largest projection of the lane's token as a signed integer
    // (the float bits: positive floats keep their order and lie above every
    // negative one), enough to tell whether the winner is positive
    int32_t pmax[TOKF];
#pragma unroll
    for (int f = 0; f < TOKF; ++f) {
        k1[f] = k2[f] = k3[f] = 0.f;
        pmax[f] = INT32_MIN;
    }
    // the key mask in a vector register, so one v_and_or builds a key from
    // the accumulator, the mask and the column (a scalar)
    uint32_t vmask;
    asm("v_mov_b32 %0, %1" : "=v"(vmask) : "s"(keymask));

    // One accumulator set: a step issues the MFMAs of tile g, parks the next
    // tile in LDS and then runs the epilogue of tile g; with three waves per
    // SIMD (at most 168 VGPRs, asked for on the kernel) the other waves'
    // matrix-core and VALU work fill the wait. (A two-set software pipeline
    // inside the wave measured no faster and holds occupancy at two.)
    f32x16 accA[TOKF];

    auto mfma_tile = [&](int g, f32x16(&acc)[TOKF]) {
        const u32x4* cur = lds[g & 1];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const f16x8 a = __builtin_bit_cast(f16x8, cur[s * kWave + lane]);
#pragma unroll
            for (int f = 0; f < TOKF; ++f)
                acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, xb[f][s],
                                                                s ? acc[f] : (f32x16){}, 0, 0, 0);
        }
    };

    // D layout: register j of lane l is row (column of R) 8*(j/4) + 4*(l/32) + j%4,
    // column (token) l%32. Key = |p| with the low mantissa bits replaced by
    // the column, one v_and_or: the sign is not in the key. The winner's sign
    // comes from pmax, the largest signed p of the token in the round (one
    // v_max3_i32 per two values): a certified winner beats every other |p| by
    // more than the key quantisation, so p > 0 exactly when pmax >= its key.
    // The key's column omits the half-wave offset 4*(l/32), which is added
    // to the three surviving keys once per round; the rest of the column,
    // tile*32 + 8*(j/4) + j%4, is wave-uniform and lives in scalar registers.
    const uint32_t half_off = (uint32_t)(4 * (lane >> 5));   // +4 columns
    auto epilogue = [&](int g, f32x16(&acc)[TOKF]) {
        const int r = __builtin_amdgcn_readfirstlane(g / ntiles);
        const int t = __builtin_amdgcn_readfirstlane(g - r * ntiles);
        const uint32_t cb = (uint32_t)(t * kHashColTile);
#pragma unroll
        for (int f = 0; f < TOKF; ++f) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const uint32_t u = __float_as_uint(acc[f][j]);
                const uint32_t col = cb + (uint32_t)(8 * (j / 4) + (j % 4));
                top3_insert(k1[f], k2[f], k3[f], __uint_as_float((u & vmask) | col));
                if (j & 1)
                    pmax[f] = max(max(pmax[f], __float_as_int(acc[f][j - 1])), (int32_t)u);
            }
        }
        if (t != ntiles - 1) return;
        const float rn_s = rbound[r], res_s = rbound[dm.nh + r];
        const float Ea = 2.f * (res_s + kAcc * rn_s), Eb = 2.f * kFlushX * rn_s;
#pragma unroll
        for (int f = 0; f < TOKF; ++f) {
            // keys are non-negative floats whose bit patterns stay below the
            // masked float part, so an integer add moves the column by 4
            k1[f] = __uint_as_float(__float_as_uint(k1[f]) + half_off);
            k2[f] = __uint_as_float(__float_as_uint(k2[f]) + half_off);
            k3[f] = __uint_as_float(__float_as_uint(k3[f]) + half_off);
            const float p1 = __shfl_xor(k1[f], 32);
            const float p2 = __shfl_xor(k2[f], 32);
            const float p3 = __shfl_xor(k3[f], 32);
            top3_insert(k1[f], k2[f], k3[f], p1);
            top3_insert(k1[f], k2[f], k3[f], p2);
            top3_insert(k1[f], k2[f], k3[f], p3);
            const float pm = __int_as_float(max(pmax[f], __shfl_xor(pmax[f], 32)));
            const bool mine = lane < 32 && tok_live[f];
            const uint32_t b1 = __float_as_uint(k1[f]), b2 = __float_as_uint(k2[f]);
            const float v1 = __uint_as_float(b1 & keymask);
            const float v2 = __uint_as_float(b2 & keymask);
            const float v3 = __uint_as_float(__float_as_uint(k3[f]) & keymask);
            const float xn = sqrtf(xn2[f]) * (1.0f + (float)(D + 4) * kTwoM24);
            const float thr = Ea * xn + Eb + v1 * qerr + 1e-30f;
            const int mode = classify(v1, v2, v3, thr);
            const int c1 = (int)(b1 & ~keymask), c2 = (int)(b2 & ~keymask);
            const int bucket = c1 < half ? c1 + (pm >= v1 ? 0 : half) : 0;
            const int32_t item = item0[f] + r * dm.L;
            if (mine) buckets[item] = bucket;
            RefineItem it{item, c1, c2, mode};
            qw.push(mine && mode >= 0, it, lane);
            k1[f] = k2[f] = k3[f] = 0.f;
            pmax[f] = INT32_MIN;
        }
    };

    // One step: start fetching tile g+2 from L2 into registers, MFMAs of tile
    // g, park tile g+1 (fetched a step ago) in the LDS buffer tile g-1 used,
    // epilogue of tile g. Two register sets keep two tiles in flight, so L2
    // latency is hidden behind a whole step.
    auto fetch = [&](int t, u32x4(&pre)[PRE]) {
        if (t < total) {
            const u32x4* src = rf + (int64_t)t * TILE_U4;
#pragma unroll
            for (int j = 0; j < PRE; ++j) pre[j] = src[threadIdx.x + j * 256];
        }
    };
    auto step = [&](int g, f32x16(&acc)[TOKF], u32x4(&pre_new)[PRE], u32x4(&pre_old)[PRE]) {
        fetch(g + 2, pre_new);
        mfma_tile(g, acc);
        if (g + 1 < total) {
            u32x4* dst = lds[(g + 1) & 1];
#pragma unroll
            for (int j = 0; j < PRE; ++j) dst[threadIdx.x + j * 256] = pre_old[j];
        }
        epilogue(g, acc);
        __syncthreads();
    };

    u32x4 preA[PRE], preB[PRE];
    fetch(1, preA);
    int g = 0;
    for (; g + 1 < total; g += 2) {
        step(g, accA, preB, preA);
        step(g + 1, accA, preA, preB);
    }
    if (g < total) step(g, accA, preB, preA);
    qw.finish(rcount, region, lane);
    refine_region(qk, rt, dm, qw.base, qw.size, qw.n0, qw.n1, lane, buckets, scount, slist, sbest,
                  cap);
}

// ------------------------------------------------------------------ fast pass (fp32 FMA)
// One thread per (token, round); the block's round is uniform so R reads are
// scalar (with per-head rotations, PH, each lane reads its own head's R).
// Used for fp32 inputs (and any dtype when requested).
template <int D, typename T, bool PH>
__global__ __launch_bounds__(256) void hash_valu_kernel(const T* __restrict__ qk,
                                                        const float* __restrict__ R,
                                                        const float* __restrict__ tnorm, Dims dm,
                                                        int32_t* __restrict__ buckets,
                                                        RefineItem* __restrict__ queue,
                                                        int32_t* __restrict__ rcount,
                                                        const float* __restrict__ rt,
                                                        int32_t* __restrict__ scount,
                                                        int32_t* __restrict__ slist,
                                                        uint64_t* __restrict__ sbest,
                                                        int64_t cap) {
    constexpr float kCoef = (float)(2 * D + 8) * kTwoM24;
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.y;
    const int half = dm.nb / 2;
    // queue region of this wave: its 64 tokens in round r
    const int64_t region = (int64_t)r * gridDim.x * 4 + (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    RegionWriter qw{queue + region * kWave, kWave, 0, 0};
    const int64_t tok = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool live = tok < dm.T;
    float x[D];
    float xn2 = 0.f;
#pragma unroll
    for (int k = 0; k < D; ++k) {
        x[k] = live ? IO<T>::load(qk, tok * D + k) : 0.f;
        xn2 = fmaf(x[k], x[k], xn2);
    }
    const int rr = (PH && live) ? r_round(dm, tok / dm.L, r) : r;   // R round
    const float* Rr = R + (int64_t)rr * D * half;
    float v1 = -1.f, v2 = -1.f, v3 = -1.f;
    int i1 = 0, i2 = 0;
    bool neg1 = false;
    for (int col = 0; col < half; ++col) {
        float p = 0.f;
#pragma unroll
        for (int k = 0; k < D; ++k) p = fmaf(x[k], Rr[(int64_t)k * half + col], p);
        const float a = fabsf(p);
        if (a > v1) {
            v3 = v2; v2 = v1; i2 = i1; v1 = a; i1 = col; neg1 = p < 0.f;
        } else if (a > v2) {
            v3 = v2; v2 = a; i2 = col;
        } else if (a > v3) {
            v3 = a;
        }
    }
    if (half == 1) { v2 = 0.f; v3 = 0.f; i2 = 0; }     // a single column: compare with -p only
    if (half == 2) v3 = 0.f;
    const float xn = sqrtf(xn2) * (1.0f + (float)(D + 4) * kTwoM24);
    const int ntiles = (half + kHashColTile - 1) / kHashColTile;
    float rn = 0.f;   // the round's largest column norm, over its tiles
    for (int i = 0; i < ntiles; ++i) rn = fmaxf(rn, tnorm[(int64_t)rr * ntiles + i]);
    const float thr = 2.f * kCoef * xn * rn + v1 * 9.5367431640625e-7f + 1e-30f;
    int mode = classify(v1, v2, v3, thr);
    if (half == 1) mode = (v1 > thr) ? -1 : 1;
    int64_t item = 0;
    if (live) {
        const int64_t bh = tok / dm.L, i = tok - bh * dm.L;
        item = (bh * dm.nh + r) * dm.L + i;
        buckets[item] = i1 + (neg1 ? half : 0);
    }
    RefineItem it{(int32_t)item, i1, i2, mode};
    qw.push(live && mode >= 0, it, lane);
    qw.finish(rcount, region, lane);
    refine_region(qk, rt, dm, qw.base, qw.size, qw.n0, qw.n1, lane, buckets, scount, slist, sbest,
                  cap);
}

// ------------------------------------------------------------------ re-decision, part 2
// Every column for the listed items of an R round, grouped so that a
// workgroup reads one 32-column tile of R once for 64 items. Block (t, r, z)
// takes groups z, z + Z, ... of R round r's list. Each (item, column) product is
// summed in fp64; the best of the tile goes into the item's key by a 64-bit
// atomic max. Key = bits of |p| (a non-negative double, so integer order is
// float order) with the low 12 bits replaced by 4095 - bucket: equal |p| then
// prefer the lower bucket index, and values closer than 2^-40 relative count
// as equal. A round of one tile (n_buckets <= 64) is all in one workgroup, so
// the item's bucket is stored at once and no finishing pass is needed.
// The extra row of blocks (y = number of R rounds) sums the queue regions'
// counts into the public count.
template <int D, typename T>
__global__ __launch_bounds__(256) void hash_scan_kernel(const T* __restrict__ qk,
                                                        const float* __restrict__ rt, Dims dm,
                                                        const int32_t* __restrict__ scount,
                                                        const int32_t* __restrict__ slist,
                                                        uint64_t* __restrict__ sbest,
                                                        int64_t cap, int32_t* __restrict__ buckets,
                                                        const int32_t* __restrict__ rcount,
                                                        int64_t nregions,
                                                        int32_t* __restrict__ counter,
                                                        int spec) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int G = 64;
    constexpr int S = D + 4;      // row stride: 16-byte aligned rows, rows 4 banks apart
    __shared__ __attribute__((aligned(16))) float rtile[kHashColTile][S];
    __shared__ __attribute__((aligned(16))) float xs[G][S];
    __shared__ int64_t xrow[G];   // element offset of each item's row of x
    __shared__ int32_t xitem[G];  // each item's flat bucket index
    // x: (column tile, group stride); y/z: R round
    const int ntiles = (dm.nb / 2 + kHashColTile - 1) / kHashColTile;
    const int t = blockIdx.x % ntiles, zg = blockIdx.x / ntiles, Z = gridDim.x / ntiles;
    const int r = (int)block_y();
    if (r > dm.nr) return;
    if (r == dm.nr) {
        // the public count: the queue regions' two counts, summed
        if (blockIdx.x != 0) return;
        __shared__ int32_t part[4];
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        int32_t c = 0;
#pragma unroll 16
        for (int64_t i = threadIdx.x; i < 2 * nregions; i += 256) c += rcount[i];
        for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
        if (lane == 0) part[wave] = c;
        __syncthreads();
        if (threadIdx.x == 0) counter[0] = part[0] + part[1] + part[2] + part[3];
        return;
    }
    const int half = dm.nb / 2;
    const int hpad = ((half + kHashColTile - 1) / kHashColTile) * kHashColTile;
    const int64_t first = (int64_t)zg * G;
    // With spec (a launch of few workgroups, each on the critical path), the
    // first group's list entries are read together with the list count
    // (entries up to the list's capacity are in bounds; those past the count
    // are never used), and its x rows are requested together with the R tile,
    // so the group starts after two dependent memory round trips, not four.
    // (In a launch of thousands of mostly idle workgroups the extra reads cost
    // more than they save.) Thread i gathers 16-byte piece i % QPR of rows
    // i / QPR + u * (256 / QPR).
    constexpr int QPR = D / 4, JPT = G * QPR / 256;
    const int j0 = threadIdx.x / QPR, kq = 4 * (threadIdx.x % QPR);
    const int32_t* lr = slist + (int64_t)r * cap;
    int32_t pit[JPT];
    int32_t myitem = 0;
    if (spec) {
#pragma unroll
        for (int u = 0; u < JPT; ++u) {
            const int64_t e = first + j0 + u * (256 / QPR);
            pit[u] = e < cap ? lr[e] : 0;
        }
        if (threadIdx.x < G && first + threadIdx.x < cap) myitem = lr[first + threadIdx.x];
    }
    const int n = min(scount[r], (int)cap);
    if (first >= n) return;
    if (!spec) {
        const float* Rt = rt + ((int64_t)r * hpad + (int64_t)t * kHashColTile) * D;
#pragma unroll 4
        for (int i = threadIdx.x; i < kHashColTile * D / 4; i += 256) {
            const int c = i / (D / 4), k = 4 * (i % (D / 4));
            *(f32x4*)&rtile[c][k] = *(const f32x4*)(Rt + (int64_t)c * D + k);
        }
    } else {
        const int gn = (int)min((int64_t)G, n - first);
        f32x4 xv[JPT];
#pragma unroll
        for (int u = 0; u < JPT; ++u) {
            const int j = j0 + u * (256 / QPR);
            xv[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
            if (j < gn) {
                const int pos = pit[u] % dm.L, bh = pit[u] / dm.L / dm.nh;
                xv[u] = IO<T>::load4(qk, ((int64_t)bh * dm.L + pos) * D + kq);
            }
        }
        const float* Rt = rt + ((int64_t)r * hpad + (int64_t)t * kHashColTile) * D;
#pragma unroll 4
        for (int i = threadIdx.x; i < kHashColTile * D / 4; i += 256) {
            const int c = i / (D / 4), k = 4 * (i % (D / 4));
            *(f32x4*)&rtile[c][k] = *(const f32x4*)(Rt + (int64_t)c * D + k);
        }
#pragma unroll
        for (int u = 0; u < JPT; ++u) *(f32x4*)&xs[j0 + u * (256 / QPR)][kq] = xv[u];
        if (threadIdx.x < G) xitem[threadIdx.x] = (int)threadIdx.x < gn ? myitem : 0;
    }
    const int it = threadIdx.x >> 2, cq = threadIdx.x & 3;   // item, column quarter
    for (int64_t g0 = first; g0 < n; g0 += (int64_t)Z * G) {
        const int gn = (int)min((int64_t)G, n - g0);
        if (g0 != first || !spec) {   // groups whose rows are not gathered yet
            __syncthreads();
            if (threadIdx.x < G) {
                int64_t off = -1;
                int32_t item = 0;
                if ((int)threadIdx.x < gn) {
                    item = lr[g0 + threadIdx.x];
                    const int pos = item % dm.L, bh = item / dm.L / dm.nh;
                    off = ((int64_t)bh * dm.L + pos) * D;
                }
                xrow[threadIdx.x] = off;
                xitem[threadIdx.x] = item;
            }
            __syncthreads();
#pragma unroll 8
            for (int i = threadIdx.x; i < G * D / 4; i += 256) {
                const int j = i / (D / 4), k = 4 * (i % (D / 4));
                const int64_t off = xrow[j];
                *(f32x4*)&xs[j][k] =
                    off >= 0 ? IO<T>::load4(qk, off + k) : (f32x4){0.f, 0.f, 0.f, 0.f};
            }
        }
        __syncthreads();
        if (it >= gn) continue;
        // The thread's columns cq, cq + 4, ..., each summed in k order in its
        // own fp64 chain; the chains are independent, so the additions of one
        // wait behind those of the others instead of behind their own.
        constexpr int NC = kHashColTile / 4;
        double p[NC];
#pragma unroll
        for (int u = 0; u < NC; ++u) p[u] = 0.0;
#pragma unroll 2
        for (int k = 0; k < D; k += 4) {
            const f32x4 a = *(const f32x4*)&xs[it][k];
#pragma unroll
            for (int u = 0; u < NC; ++u) {
                const f32x4 b = *(const f32x4*)&rtile[cq + 4 * u][k];
#pragma unroll
                for (int e = 0; e < 4; ++e) p[u] += (double)a[e] * (double)b[e];
            }
        }
        uint64_t best = 0;
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const int col = t * kHashColTile + cq + 4 * u;
            if (col < half) {
                const int bucket = col + (p[u] < 0.0 ? half : 0);
                const uint64_t key = (__double_as_longlong(fabs(p[u])) & ~0xFFFull) |
                                     (uint64_t)(4095 - bucket);
                best = key > best ? key : best;
            }
        }
        for (int off = 1; off < 4; off <<= 1) {
            const uint64_t o = __shfl_xor(best, off);
            best = o > best ? o : best;
        }
        if (cq == 0) {
            if (ntiles == 1)
                buckets[xitem[it]] = 4095 - (int)(best & 0xFFFull);
            else
                atomicMax((unsigned long long*)&sbest[(int64_t)r * cap + g0 + it], best);
        }
    }
}

// The listed items take the bucket of their best key (rounds of more than one
// column tile, whose tiles were scanned by different workgroups).
__global__ __launch_bounds__(256) void hash_scan_finish_kernel(const int32_t* __restrict__ scount,
                                                               const int32_t* __restrict__ slist,
                                                               const uint64_t* __restrict__ sbest,
                                                               int64_t cap, int nr,
                                                               int32_t* __restrict__ buckets) {
    const int r = (int)block_y();   // R round
    if (r >= nr) return;
    const int n = min(scount[r], (int)cap);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        buckets[slist[(int64_t)r * cap + i]] = 4095 - (int)(sbest[(int64_t)r * cap + i] & 0xFFFull);
}

// ------------------------------------------------------------------ launcher
template <typename T>
static hipError_t launch_scan(const T* qk, const Dims& d, int32_t* buckets, const HashWorkspace& w,
                              int64_t nregions, hipStream_t st, hipEvent_t* ev, int* nev,
                              const char** names) {
    const int64_t cap = queue_tokens(d);
    // enough groups for a few thousand listed items per round; more loop
    const unsigned z = (unsigned)std::min<int64_t>(16, (cap + 63) / 64);
    // one row of blocks per R round, and one more for the public count
    const dim3 sgrid = grid_split((unsigned)hash_ntiles(d) * z, (int64_t)d.nr + 1);
    // prefetch the first group when the launch is small (at most 512 blocks)
    const int spec = (int64_t)hash_ntiles(d) * z * d.nr <= 512;
    if (d.d == 64)
        hash_scan_kernel<64, T><<<sgrid, 256, 0, st>>>(qk, w.rt, d, w.scount, w.slist, w.sbest, cap,
                                                       buckets, w.rcount, nregions, w.counter,
                                                       spec);
    else
        hash_scan_kernel<128, T><<<sgrid, 256, 0, st>>>(qk, w.rt, d, w.scount, w.slist, w.sbest,
                                                        cap, buckets, w.rcount, nregions,
                                                        w.counter, spec);
    if (hash_ntiles(d) > 1)
        hash_scan_finish_kernel<<<grid_split(4, d.nr), 256, 0, st>>>(w.scount, w.slist, w.sbest,
                                                                     cap, d.nr, buckets);
    return mark(st, ev, nev, names, "hash_refine_scan");
}

hipError_t launch_hash(const void* qk, const float* R, const Dims& d, int32_t* buckets,
                       const HashWorkspace& w, hipStream_t st, hipEvent_t* ev, int* nev,
                       const char** names, const void* v_for_max) {
    const int half = d.nb / 2;
    const int ntiles = hash_ntiles(d);
    hipError_t e;
    const dim3 pgrid = grid_split((unsigned)ntiles, d.nr);   // every R round
    if (ntiles == 1)
        rprep_kernel<true><<<pgrid, 256, 0, st>>>(R, d.d, half, ntiles, d.nr, w.tnorm, w.rt,
                                                  w.rfrag, w.counter, w.scount);
    else
        rprep_kernel<false><<<pgrid, 256, 0, st>>>(R, d.d, half, ntiles, d.nr, w.tnorm, w.rt,
                                                   w.rfrag, w.counter, w.scount);
    if ((e = mark(st, ev, nev, names, "hash_prep")) != hipSuccess) return e;
    if (d.dtype == LSH_BF16) {
        // two 32-token fragments per wave (32 and 128 tokens per wave measured
        // slower)
        constexpr int TOKF = 2;
        constexpr int per_wave = 32 * TOKF, per_wg = 4 * per_wave;
        static_assert(per_wg <= kQueuePad && kQueuePad % per_wg == 0,
                      "queue regions must fit the padded capacity");
        static_assert(per_wave >= kWave, "the re-decision pass reads 64 entries of a region ahead");
        // with per-head rotations each (batch, head) starts a new workgroup
        const unsigned grid = d.per_head_r
                                  ? (unsigned)((int64_t)d.B * d.H * ((d.L + per_wg - 1) / per_wg))
                                  : (unsigned)((d.T + per_wg - 1) / per_wg);
        const uint16_t* x = (const uint16_t*)qk;
        const size_t rb_lds = sizeof(float) * 2 * d.nh;   // per-round bounds
        const int64_t cap = queue_tokens(d);
        if (d.d == 64)
            hash_mfma_kernel<64, TOKF><<<grid, 256, rb_lds, st>>>(
                x, (const u32x4*)w.rfrag, w.tnorm, d, buckets, w.queue, w.rcount,
                (const uint16_t*)v_for_max, w.vmax, w.rt, w.scount, w.slist, w.sbest, cap);
        else
            hash_mfma_kernel<128, TOKF><<<grid, 256, rb_lds, st>>>(
                x, (const u32x4*)w.rfrag, w.tnorm, d, buckets, w.queue, w.rcount,
                (const uint16_t*)v_for_max, w.vmax, w.rt, w.scount, w.slist, w.sbest, cap);
        if ((e = mark(st, ev, nev, names, "hash_fast_mfma")) != hipSuccess) return e;
        return launch_scan(x, d, buckets, w, (int64_t)grid * 4, st, ev, nev, names);
    } else {
        const float* x = (const float*)qk;
        dim3 grid((unsigned)((d.T + 255) / 256), (unsigned)d.nh);
        const int64_t cap = queue_tokens(d);
#define LSH_HASH_VALU(DD, PH)                                                                  \
    hash_valu_kernel<DD, float, PH><<<grid, 256, 0, st>>>(x, R, w.tnorm, d, buckets, w.queue,   \
                                                          w.rcount, w.rt, w.scount, w.slist,   \
                                                          w.sbest, cap)
        if (d.d == 64) {
            if (d.per_head_r) LSH_HASH_VALU(64, true);
            else LSH_HASH_VALU(64, false);
        } else {
            if (d.per_head_r) LSH_HASH_VALU(128, true);
            else LSH_HASH_VALU(128, false);
        }
#undef LSH_HASH_VALU
        if ((e = mark(st, ev, nev, names, "hash_fast_fp32")) != hipSuccess) return e;
        return launch_scan(x, d, buckets, w, (int64_t)grid.x * 4 * d.nh, st, ev, nev, names);
    }
}

}  // namespace lsh
