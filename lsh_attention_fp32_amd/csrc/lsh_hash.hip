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
//  * Fast pass on the matrix cores. R is split exactly enough into two bf16
//    terms, R = r_hi + r_lo + e with |e| <= 2^-16 |R|; with bf16 inputs every
//    product x*r is exact in fp32 and the MFMA accumulates in fp32. Each lane
//    keeps the three largest |p| of its token as packed keys (|p| with the low
//    mantissa bits replaced by (column << 1 | sign)), three integer min/max
//    operations per value.
//  * Certification. With the Cauchy-Schwarz bound sum_k |x_k R_kb| <=
//    |x| |R_b|, every fast value is within E = coef * |x| * max_b |R_b| of the
//    exact one. If the top key beats the second by more than 2E (plus the key
//    quantisation), the bucket is the exact argmax. If only the third is
//    certainly out, the token-round is queued with its two candidate columns;
//    otherwise with a request to scan every column.
//  * Re-decision in fp64 on the GPU for the queued token-rounds (typically a
//    fraction of a percent).
//  * fp32 inputs (or head sizes without a matrix-core kernel) use a plain fp32
//    FMA pass with the same certification and re-decision.
#include <algorithm>

#include "lsh_internal.h"

namespace lsh {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

static constexpr float kTwoM24 = 5.9604644775390625e-8f;   // 2^-24

// ------------------------------------------------------------------ workspace
static size_t rfrag_elems(const Dims& d) {
    // [nh][ntiles][d/16 k-steps][2 splits][64 lanes][8] bf16
    return (size_t)d.nh * hash_ntiles(d) * kHashColTile * d.d * 2;
}

static size_t rt_elems(const Dims& d) {
    // [nh][ntiles * 32 columns][d] float32
    return (size_t)d.nh * hash_ntiles(d) * kHashColTile * d.d;
}

size_t hash_workspace_bytes(const Dims& d) {
    size_t b = 256;                                              // counter
    b += align_up(sizeof(float) * d.nh, 256);                    // rnorm
    b += align_up(sizeof(uint16_t) * rfrag_elems(d), 256);       // rfrag
    b += align_up(sizeof(float) * rt_elems(d), 256);             // rt
    b += align_up(sizeof(RefineItem) * (size_t)d.T * d.nh, 256); // queue
    return b;
}

HashWorkspace carve_hash_workspace(void* ws, const Dims& d) {
    char* p = (char*)ws;
    HashWorkspace w;
    w.counter = (int32_t*)p;
    w.vmax = (uint32_t*)(p + 3 * sizeof(int32_t));
    p += 256;
    w.rnorm = (float*)p;
    p += align_up(sizeof(float) * d.nh, 256);
    w.rfrag = (uint16_t*)p;
    p += align_up(sizeof(uint16_t) * rfrag_elems(d), 256);
    w.rt = (float*)p;
    p += align_up(sizeof(float) * rt_elems(d), 256);
    w.queue = (RefineItem*)p;
    return w;
}

// ------------------------------------------------------------------ R prep
__global__ void zero_counter_kernel(int32_t* counter, float* rnorm, int nh) {
    if (threadIdx.x < 4) counter[threadIdx.x] = 0;   // three queue counters and max|v|
    for (int r = threadIdx.x; r < nh; r += blockDim.x) rnorm[r] = 0.f;
}

// One workgroup per (round, 32-column tile) of R, staged through LDS:
//  * rnorm[r]  = max over columns of |R[r, :, col]|_2, rounded up (atomic max on
//               the bits of a non-negative float, order independent);
//  * rt        = R transposed to [round][column][k] in fp32 (padded columns are 0),
//               read by the fp64 re-decision;
//  * rfrag     = the bf16 hi/lo split of R in the A-operand order of
//               v_mfma_f32_32x32x16_bf16: for (round, tile, k-step, split), 64
//               lanes of 8 values, lane l holding column tile*32 + l%32 and
//               k = kstep*16 + 8*(l/32) + e.
__global__ __launch_bounds__(256) void rprep_kernel(const float* __restrict__ R, int d, int half,
                                                    int ntiles, float* __restrict__ rnorm,
                                                    float* __restrict__ rt,
                                                    uint16_t* __restrict__ rfrag) {
    __shared__ float tile[128][kHashColTile + 1];
    const int t = blockIdx.x, r = blockIdx.y;
    const int col0 = t * kHashColTile;
    for (int idx = threadIdx.x; idx < d * kHashColTile; idx += 256) {
        const int k = idx / kHashColTile, c = idx % kHashColTile;
        tile[k][c] = (col0 + c < half) ? R[((int64_t)r * d + k) * half + col0 + c] : 0.f;
    }
    __syncthreads();
    if (threadIdx.x < kHashColTile) {
        float ss = 0.f;
        for (int k = 0; k < d; ++k) ss = fmaf(tile[k][threadIdx.x], tile[k][threadIdx.x], ss);
        // fp32 sum of d squares: relative error below d * 2^-24; sqrt halves it
        const float nrm = sqrtf(ss) * (1.0f + (float)(d + 4) * kTwoM24);
        atomicMax((int*)&rnorm[r], __float_as_int(nrm));
    }
    float* dst = rt + ((int64_t)r * ntiles * kHashColTile + col0) * d;
    for (int idx = threadIdx.x; idx < d * kHashColTile; idx += 256) {
        const int c = idx / d, k = idx % d;
        dst[idx] = tile[k][c];
    }
    const int ks = d / 16;
    for (int f = threadIdx.x; f < ks * 2 * kWave; f += 256) {
        const int lane = f & 63, q = (f >> 6) & 1, s = f >> 7;
        const int c = lane & 31, k0 = s * 16 + 8 * (lane >> 5);
        uint32_t w[4];
        for (int e2 = 0; e2 < 4; ++e2) {
            uint32_t pair = 0;
            for (int h = 0; h < 2; ++h) {
                const float val = tile[k0 + 2 * e2 + h][c];
                const uint16_t hi = f32_to_bf16(val);
                const uint16_t lo = f32_to_bf16(val - bf16_to_f32(hi));  // the difference is exact
                pair |= (uint32_t)(q ? lo : hi) << (16 * h);
            }
            w[e2] = pair;
        }
        u32x4 pk = {w[0], w[1], w[2], w[3]};
        *(u32x4*)(rfrag + ((((int64_t)r * ntiles + t) * ks * 2 + f / kWave) * kWave + lane) * 8) = pk;
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

// Appends the flagged lanes' items to the queue, one atomic per wave and mode.
// The queue has room for every token-round; two-candidate items (mode 0) fill
// it from the front, full scans (mode 1) from the back. counter[0] counts all
// items, counter[1] the front part, counter[2] the back part.
__device__ __forceinline__ void queue_push(bool flag, RefineItem it, int32_t* counter,
                                           RefineItem* queue, int capacity, int lane) {
    const uint64_t any = __ballot(flag);
    if (!any) return;
    const uint64_t m1 = __ballot(flag && it.mode == 1);
    const uint64_t m0 = any & ~m1;
    const int leader = __ffsll((long long)any) - 1;
    int b0 = 0, b1 = 0;
    if (lane == leader) {
        atomicAdd(&counter[0], __popcll(any));
        if (m0) b0 = atomicAdd(&counter[1], __popcll(m0));
        if (m1) b1 = atomicAdd(&counter[2], __popcll(m1));
    }
    b0 = __shfl(b0, leader);
    b1 = __shfl(b1, leader);
    if (!flag) return;
    if (it.mode == 1)
        queue[capacity - 1 - (b1 + __popcll(m1 & lanes_below(lane)))] = it;
    else
        queue[b0 + __popcll(m0 & lanes_below(lane))] = it;
}

// Decision shared by both fast passes. v1 >= v2 >= v3 are the three largest
// fast |p| values (as floats), thr the certification threshold.
__device__ __forceinline__ int classify(float v1, float v2, float v3, float thr) {
    if (v1 - v2 > thr) return -1;  // certified
    if (v1 - v3 > thr) return 0;   // two candidates
    return 1;                      // scan every column
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
__global__ __launch_bounds__(256) void hash_mfma_kernel(const uint16_t* __restrict__ qk,
                                                        const u32x4* __restrict__ rfrag,
                                                        const float* __restrict__ rnorm, Dims dm,
                                                        int32_t* __restrict__ buckets,
                                                        int32_t* __restrict__ counter,
                                                        RefineItem* __restrict__ queue,
                                                        const uint16_t* __restrict__ v,
                                                        uint32_t* __restrict__ vmax) {
    constexpr int KS = D / 16;
    constexpr int TILE_U4 = KS * 2 * kWave;     // 16-byte lane fragments per column tile
    constexpr int PRE = TILE_U4 / 256;          // fragments each thread stages
    constexpr int TOK_WAVE = 32 * TOKF;
    constexpr int TOK_WG = 4 * TOK_WAVE;
    constexpr float kCoef = (float)(4 * D + 8) * kTwoM24 + 3.0517578125e-5f;  // + 2^-15
    __shared__ u32x4 lds[2][TILE_U4];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = dm.nb / 2;
    const int capacity = (int)(dm.T * dm.nh);
    const int ntiles = (half + kHashColTile - 1) / kHashColTile;
    const int total = dm.nh * ntiles;
    const int64_t tok0 = (int64_t)blockIdx.x * TOK_WG + (int64_t)wave * TOK_WAVE;
    const int bits = 32 - __clz(2 * ntiles * kHashColTile - 1);
    const uint32_t keymask = 0x7FFFFFFFu & ~((1u << bits) - 1u);
    const float qerr = __uint_as_float((uint32_t)(127 + bits - 22) << 23) + 9.5367431640625e-7f;

    // B operand: lane holds x[tok0 + f*32 + lane%32][16 s + 8 (lane/32) + e]
    bf16x8 xb[TOKF][KS];
    float xn2[TOKF];
#pragma unroll
    for (int f = 0; f < TOKF; ++f) {
        const int64_t tok = tok0 + f * 32 + (lane & 31);
        xn2[f] = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 u = {0u, 0u, 0u, 0u};
            if (tok < dm.T) u = ((const u32x4*)(qk + tok * D))[2 * s + (lane >> 5)];
            xb[f][s] = __builtin_bit_cast(bf16x8, u);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = __uint_as_float(u[e] << 16), b = __uint_as_float(u[e] & 0xFFFF0000u);
                xn2[f] = fmaf(a, a, fmaf(b, b, xn2[f]));
            }
        }
        xn2[f] += __shfl_xor(xn2[f], 32);
    }
    // flat index of (token, round 0) in buckets [B,H,nh,L]; round r adds r*L
    int32_t item0[TOKF];
    bool tok_live[TOKF];
#pragma unroll
    for (int f = 0; f < TOKF; ++f) {
        const int64_t tok = tok0 + f * 32 + (lane & 31);
        tok_live[f] = tok < dm.T;
        const int64_t bh = tok / dm.L, i = tok - bh * dm.L;
        item0[f] = tok_live[f] ? (int32_t)(bh * dm.nh * dm.L + i) : 0;
    }

    __shared__ uint32_t wvmax[4];
    if (v) {
        // this workgroup's tokens are one contiguous run of value rows
        const int64_t first = (int64_t)blockIdx.x * TOK_WG;
        const int64_t nvec = min((int64_t)TOK_WG, dm.T - first) * (D / 8);
        const u32x4* src = (const u32x4*)(v + first * D);
        uint32_t m = 0;
        for (int64_t i = threadIdx.x; i < nvec; i += 256) {
            const u32x4 w = src[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) m = max(m, max(w[e] & 0x7FFFu, (w[e] >> 16) & 0x7FFFu));
        }
        for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
        if (lane == 0) wvmax[wave] = m;
    }
    for (int i = threadIdx.x; i < TILE_U4; i += 256) lds[0][i] = rfrag[i];
    __syncthreads();
    if (v && threadIdx.x == 0)
        atomicMax(vmax, max(max(wvmax[0], wvmax[1]), max(wvmax[2], wvmax[3])));

    float k1[TOKF], k2[TOKF], k3[TOKF];
#pragma unroll
    for (int f = 0; f < TOKF; ++f) k1[f] = k2[f] = k3[f] = 0.f;

    // Software pipeline: the MFMAs of tile g are issued before the epilogue of
    // tile g-1, which reads the other accumulator set, so the wave's VALU work
    // overlaps its own matrix-core work.
    f32x16 accA[TOKF], accB[TOKF];

    auto mfma_tile = [&](int g, f32x16(&acc)[TOKF]) {
        const u32x4* cur = lds[g & 1];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 ahi = __builtin_bit_cast(bf16x8, cur[(2 * s + 0) * kWave + lane]);
            const bf16x8 alo = __builtin_bit_cast(bf16x8, cur[(2 * s + 1) * kWave + lane]);
#pragma unroll
            for (int f = 0; f < TOKF; ++f) {
                acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, xb[f][s],
                                                                 s ? acc[f] : (f32x16){}, 0, 0, 0);
                acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, xb[f][s], acc[f], 0, 0, 0);
            }
        }
    };

    // D layout: register j of lane l is row (column of R) 8*(j/4) + 4*(l/32) + j%4,
    // column (token) l%32. Key = |p| with the low mantissa bits replaced by
    // (column << 1 | sign): alignbit builds the index, and_or merges it.
    // The key's column omits the half-wave offset 4*(l/32), which is added to the
    // three surviving keys once per round; the rest of the column, tile*32 +
    // 8*(j/4) + j%4, is wave-uniform and lives in scalar registers.
    const float half_off = __uint_as_float((uint32_t)(8 * (lane >> 5)));   // +4 columns
    auto epilogue = [&](int g, f32x16(&acc)[TOKF]) {
        const int r = __builtin_amdgcn_readfirstlane(g / ntiles);
        const int t = __builtin_amdgcn_readfirstlane(g - r * ntiles);
        const uint32_t cb = (uint32_t)(t * kHashColTile);
#pragma unroll
        for (int f = 0; f < TOKF; ++f) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const uint32_t u = __float_as_uint(acc[f][j]);
                const uint32_t idx =
                    __builtin_amdgcn_alignbit(cb + (uint32_t)(8 * (j / 4) + (j % 4)), u, 31);
                top3_insert(k1[f], k2[f], k3[f], __uint_as_float((u & keymask) | idx));
            }
        }
        if (t != ntiles - 1) return;
        const float E2 = 2.f * kCoef * rnorm[r];
#pragma unroll
        for (int f = 0; f < TOKF; ++f) {
            // keys are non-negative floats whose bit patterns stay below the
            // masked float part, so an integer add moves the column by 4
            k1[f] = __uint_as_float(__float_as_uint(k1[f]) + __float_as_uint(half_off));
            k2[f] = __uint_as_float(__float_as_uint(k2[f]) + __float_as_uint(half_off));
            k3[f] = __uint_as_float(__float_as_uint(k3[f]) + __float_as_uint(half_off));
            const float p1 = __shfl_xor(k1[f], 32);
            const float p2 = __shfl_xor(k2[f], 32);
            const float p3 = __shfl_xor(k3[f], 32);
            top3_insert(k1[f], k2[f], k3[f], p1);
            top3_insert(k1[f], k2[f], k3[f], p2);
            top3_insert(k1[f], k2[f], k3[f], p3);
            const bool mine = lane < 32 && tok_live[f];
            const uint32_t b1 = __float_as_uint(k1[f]), b2 = __float_as_uint(k2[f]);
            const float v1 = __uint_as_float(b1 & keymask);
            const float v2 = __uint_as_float(b2 & keymask);
            const float v3 = __uint_as_float(__float_as_uint(k3[f]) & keymask);
            const float xn = sqrtf(xn2[f]) * (1.0f + (float)(D + 4) * kTwoM24);
            const float thr = E2 * xn + v1 * qerr + 1e-30f;
            const int mode = classify(v1, v2, v3, thr);
            const uint32_t i1 = b1 & ~keymask & 0x7FFFFFFFu, i2 = b2 & ~keymask & 0x7FFFFFFFu;
            const int c1 = (int)(i1 >> 1), c2 = (int)(i2 >> 1);
            const int bucket = c1 < half ? c1 + ((i1 & 1u) ? half : 0) : 0;
            const int32_t item = item0[f] + r * dm.L;
            if (mine) buckets[item] = bucket;
            RefineItem it{item, c1, c2, mode};
            queue_push(mine && mode >= 0, it, counter, queue, capacity, lane);
            k1[f] = k2[f] = k3[f] = 0.f;
        }
    };

    // One pipeline step: start fetching tile g+2 from L2 into registers, MFMAs
    // of tile g, epilogue of tile g-1, then park tile g+1 (fetched a step ago)
    // in the LDS buffer tile g-1 used. Two register sets keep two tiles in
    // flight, so L2 latency is hidden behind a whole step.
    auto fetch = [&](int t, u32x4(&pre)[PRE]) {
        if (t < total) {
            const u32x4* src = rfrag + (int64_t)t * TILE_U4;
#pragma unroll
            for (int j = 0; j < PRE; ++j) pre[j] = src[threadIdx.x + j * 256];
        }
    };
    auto step = [&](int g, f32x16(&acc_new)[TOKF], f32x16(&acc_old)[TOKF], u32x4(&pre_new)[PRE],
                    u32x4(&pre_old)[PRE]) {
        fetch(g + 2, pre_new);
        mfma_tile(g, acc_new);
        if (g > 0) epilogue(g - 1, acc_old);
        if (g + 1 < total) {
            u32x4* dst = lds[(g + 1) & 1];
#pragma unroll
            for (int j = 0; j < PRE; ++j) dst[threadIdx.x + j * 256] = pre_old[j];
        }
        __syncthreads();
    };

    u32x4 preA[PRE], preB[PRE];
    fetch(1, preA);
    step(0, accA, accB, preB, preA);
    int g = 1;
    for (; g + 1 < total; g += 2) {
        step(g, accB, accA, preA, preB);
        step(g + 1, accA, accB, preB, preA);
    }
    if (g < total) {
        step(g, accB, accA, preA, preB);
        epilogue(g, accB);
    } else {
        epilogue(g - 1, accA);
    }
}

// ------------------------------------------------------------------ fast pass (fp32 FMA)
// One thread per (token, round); the block's round is uniform so R reads are
// scalar. Used for fp32 inputs (and any dtype when requested).
template <int D, typename T>
__global__ __launch_bounds__(256) void hash_valu_kernel(const T* __restrict__ qk,
                                                        const float* __restrict__ R,
                                                        const float* __restrict__ rnorm, Dims dm,
                                                        int32_t* __restrict__ buckets,
                                                        int32_t* __restrict__ counter,
                                                        RefineItem* __restrict__ queue) {
    constexpr float kCoef = (float)(2 * D + 8) * kTwoM24;
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.y;
    const int half = dm.nb / 2;
    const int capacity = (int)(dm.T * dm.nh);
    const int64_t tok = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool live = tok < dm.T;
    float x[D];
    float xn2 = 0.f;
#pragma unroll
    for (int k = 0; k < D; ++k) {
        x[k] = live ? IO<T>::load(qk, tok * D + k) : 0.f;
        xn2 = fmaf(x[k], x[k], xn2);
    }
    const float* Rr = R + (int64_t)r * D * half;
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
    const float thr = 2.f * kCoef * xn * rnorm[r] + v1 * 9.5367431640625e-7f + 1e-30f;
    int mode = classify(v1, v2, v3, thr);
    if (half == 1) mode = (v1 > thr) ? -1 : 1;
    int64_t item = 0;
    if (live) {
        const int64_t bh = tok / dm.L, i = tok - bh * dm.L;
        item = (bh * dm.nh + r) * dm.L + i;
        buckets[item] = i1 + (neg1 ? half : 0);
    }
    RefineItem it{(int32_t)item, i1, i2, mode};
    queue_push(live && mode >= 0, it, counter, queue, capacity, lane);
}

// ------------------------------------------------------------------ re-decision in fp64
// One wave per queued token-round. Mode 0 computes the two candidate columns
// (half a wave each); mode 1 scans every column. The exact rule: largest |p|,
// ties to the lowest index of [p, -p] (a p of either zero sign counts as "+").
template <typename T>
__global__ __launch_bounds__(256) void hash_refine_kernel(const T* __restrict__ qk,
                                                          const float* __restrict__ rt, Dims dm,
                                                          const int32_t* __restrict__ counter,
                                                          const RefineItem* __restrict__ queue,
                                                          int32_t* __restrict__ buckets) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = dm.nb / 2;
    const int hpad = ((half + kHashColTile - 1) / kHashColTile) * kHashColTile;
    const int D = dm.d;
    const int capacity = (int)(dm.T * dm.nh);
    const int n0 = counter[1], n1 = counter[2];

    auto locate = [&](int32_t item, const T*& x, const float*& Rr) {
        const int i = item % dm.L;
        const int rest = item / dm.L;
        const int r = rest % dm.nh;
        const int bh = rest / dm.nh;
        x = qk + ((int64_t)bh * dm.L + i) * D;
        Rr = rt + (int64_t)r * hpad * D;      // [column][k]
    };

    // two candidate columns: one wave per item, half a wave per column
    const int64_t gwave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t q = gwave; q < n0; q += nwaves) {
        const RefineItem it = queue[q];
        const T* x;
        const float* Rr;
        locate(it.item, x, Rr);
        const int col = (lane < 32) ? it.a : it.b;
        double acc = 0.0;
        if (col >= 0 && col < half) {
            const float* rc = Rr + (int64_t)col * D;
            for (int k = lane & 31; k < D; k += 32) acc += (double)IO<T>::load(x, k) * (double)rc[k];
        }
        for (int off = 16; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        const double pa = __shfl(acc, 0), pb = __shfl(acc, 32);
        if (lane == 0) {
            const bool va = it.a >= 0 && it.a < half, vb = it.b >= 0 && it.b < half && it.b != it.a;
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

    // every column: one workgroup per item; 32 groups of 8 lanes each take a
    // column per pass, each lane an eighth of the row (16-byte loads).
    __shared__ double sv[4];
    __shared__ int si[4];
    const int part = lane & 7, grp = threadIdx.x >> 3;      // 32 column groups
    const int klen = D / 8;
    for (int64_t q = blockIdx.x; q < n1; q += gridDim.x) {
        const RefineItem it = queue[capacity - 1 - q];
        const T* x;
        const float* Rr;
        locate(it.item, x, Rr);
        double xk[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) xk[k] = k < klen ? (double)IO<T>::load(x, part * klen + k) : 0.0;
        double bestv = -1.0;
        int besti = 0x7FFFFFFF;
        for (int col0 = 0; col0 < half; col0 += 32) {
            const int col = col0 + grp;
            double p = 0.0;
            if (col < half) {
                const f32x4* rc = (const f32x4*)(Rr + (int64_t)col * D + part * klen);
                f32x4 rv[4];
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4)
                    if (4 * v4 < klen) rv[v4] = rc[v4];
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4)
                    if (4 * v4 < klen)
#pragma unroll
                        for (int e = 0; e < 4; ++e) p += xk[4 * v4 + e] * (double)rv[v4][e];
            }
            p += __shfl_xor(p, 1);
            p += __shfl_xor(p, 2);
            p += __shfl_xor(p, 4);
            if (col < half) {
                const double v = fabs(p);
                const int ci = col + (p < 0.0 ? half : 0);
                if (v > bestv || (v == bestv && ci < besti)) { bestv = v; besti = ci; }
            }
        }
        for (int off = 32; off > 0; off >>= 1) {
            const double ov = __shfl_xor(bestv, off);
            const int oi = __shfl_xor(besti, off);
            if (ov > bestv || (ov == bestv && oi < besti)) { bestv = ov; besti = oi; }
        }
        if (lane == 0) {
            sv[wave] = bestv;
            si[wave] = besti;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int w = 1; w < 4; ++w)
                if (sv[w] > bestv || (sv[w] == bestv && si[w] < besti)) { bestv = sv[w]; besti = si[w]; }
            buckets[it.item] = besti;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ launcher
template <typename T>
static hipError_t launch_valu_and_refine(const T* qk, const float* R, const Dims& d,
                                         int32_t* buckets, const HashWorkspace& w, hipStream_t st,
                                         hipEvent_t* ev, int* nev, const char** names) {
    dim3 grid((unsigned)((d.T + 255) / 256), (unsigned)d.nh);
    if (d.d == 64)
        hash_valu_kernel<64, T><<<grid, 256, 0, st>>>(qk, R, w.rnorm, d, buckets, w.counter, w.queue);
    else
        hash_valu_kernel<128, T><<<grid, 256, 0, st>>>(qk, R, w.rnorm, d, buckets, w.counter, w.queue);
    hipError_t e = mark(st, ev, nev, names, "hash_fast_fp32");
    if (e != hipSuccess) return e;
    return hipSuccess;
}

hipError_t launch_hash(const void* qk, const float* R, const Dims& d, int32_t* buckets,
                       const HashWorkspace& w, hipStream_t st, hipEvent_t* ev, int* nev,
                       const char** names, const void* v_for_max) {
    const int half = d.nb / 2;
    const int ntiles = hash_ntiles(d);
    hipError_t e;
    zero_counter_kernel<<<1, 256, 0, st>>>(w.counter, w.rnorm, d.nh);
    rprep_kernel<<<dim3((unsigned)ntiles, (unsigned)d.nh), 256, 0, st>>>(R, d.d, half, ntiles,
                                                                         w.rnorm, w.rt, w.rfrag);
    if ((e = mark(st, ev, nev, names, "hash_prep")) != hipSuccess) return e;
    // enough waves that a typical queue is drained in one or two items per wave
    const unsigned refine_blocks = (unsigned)std::min<int64_t>(4096, (d.T * d.nh + 255) / 256 + 1);
    if (d.dtype == LSH_BF16) {
#ifndef LSH_HASH_TOKF
#define LSH_HASH_TOKF 2
#endif
        constexpr int TOKF = LSH_HASH_TOKF;
        const int64_t per_wg = 4 * 32 * TOKF;
        const unsigned grid = (unsigned)((d.T + per_wg - 1) / per_wg);
        const uint16_t* x = (const uint16_t*)qk;
        if (d.d == 64)
            hash_mfma_kernel<64, TOKF><<<grid, 256, 0, st>>>(x, (const u32x4*)w.rfrag, w.rnorm, d,
                                                           buckets, w.counter, w.queue,
                                                           (const uint16_t*)v_for_max, w.vmax);
        else
            hash_mfma_kernel<128, TOKF><<<grid, 256, 0, st>>>(x, (const u32x4*)w.rfrag, w.rnorm, d,
                                                            buckets, w.counter, w.queue,
                                                            (const uint16_t*)v_for_max, w.vmax);
        if ((e = mark(st, ev, nev, names, "hash_fast_mfma")) != hipSuccess) return e;
        hash_refine_kernel<uint16_t><<<refine_blocks, 256, 0, st>>>(x, w.rt, d, w.counter, w.queue,
                                                                    buckets);
    } else {
        e = launch_valu_and_refine((const float*)qk, R, d, buckets, w, st, ev, nev, names);
        if (e != hipSuccess) return e;
        hash_refine_kernel<float><<<refine_blocks, 256, 0, st>>>((const float*)qk, w.rt, d,
                                                                 w.counter, w.queue, buckets);
    }
    return mark(st, ev, nev, names, "hash_refine_fp64");
}

}  // namespace lsh
