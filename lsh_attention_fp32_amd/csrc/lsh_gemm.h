// lsh_gemm.h -- the dense products of the library: C = out(A W^T), A [M][K]
// (token rows), W [N][K] (output-major, the layout of a linear layer's
// weight), with the output step (a bias, an activation, where each output
// goes) supplied by the caller. Used by the input projections and by the
// feed-forward.
//
// bf16: out^T = W A^T on v_mfma_f32_32x32x16_bf16 (A operand = weight rows,
// B operand = token rows: both are read along k, so every operand fragment is
// one 16-byte piece of a row), fp32 accumulation. fp32: an LDS-tiled vector
// kernel.
#pragma once

#include "lsh_internal.h"

namespace lsh {
namespace gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kPN = 256;        // outputs (n) per workgroup
constexpr int kPM = 128;        // tokens (m) per workgroup
constexpr int kPK = 32;         // k per LDS stage: a 64-byte row of four 16-byte pieces
constexpr int kXcds = 8;        // L2 domains the dispatcher deals workgroups over

// LDS rows are unpadded; piece q of row r sits at piece q ^ swz(r). A
// fragment read takes one piece of 16 consecutive rows, which then cover all
// 64 banks; a stage store writes 4 whole rows (256 contiguous bytes).
struct Lds {
    uint16_t a[2][kPN][kPK];   // weight rows
    uint16_t b[2][kPM][kPK];   // token rows
};
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// Waves per workgroup: 8, a 4 x 2 grid of waves with 64 outputs x 64 tokens
// each (four waves per SIMD hide more of the fragment-read stalls than four
// waves of 128 x 64).
constexpr int kGW = 8;
constexpr int kGT = 64 * kGW;            // threads per workgroup
constexpr int kWN = kGW / 2;             // waves along the outputs
constexpr int kNB = kPN / (32 * kWN);    // 32 x 32 blocks per wave along the outputs
constexpr int kMB = kPM / (32 * 2);      // and along the tokens
constexpr int kRows = kGT / 4;           // rows a staging pass covers (4 pieces each)
constexpr int kAL = kPN / kRows, kBL = kPM / kRows;   // weight / token loads per thread

// Weight rows n < nsplit come from w0, the others from w1 (row n - nsplit):
// two weight tensors act as one concatenated W.
struct Weights {
    const void* w0;
    const void* w1;
    int nsplit;
    template <typename T>
    __device__ __forceinline__ const T* row(int n, int K) const {
        return n < nsplit ? (const T*)w0 + (int64_t)n * K : (const T*)w1 + (int64_t)(n - nsplit) * K;
    }
};

// Output step contract (Out):
//   float act(float acc, int n)      -- the value output n stores
//   T* at(int64_t m, int n)          -- where output n of token m goes; for
//                                       n % 8 == 0 the 8 outputs n .. n+7
//                                       are contiguous (bf16 path)

// Workgroups are dealt round-robin over the L2 domains (id % kXcds). Each
// domain takes groups of kGM token tiles x kGN output tiles, so the
// workgroups it runs together share 8 token panels and 4 weight panels
// (2 + 2 MiB at K = 1024) in its L2 instead of streaming a whole weight
// matrix past each token tile.
constexpr int kGM = 8, kGN = 4;

// Workgroups to launch for ntn x ntm tiles (whole groups, every domain).
inline int64_t mfma_grid(int ntn, int64_t ntm) {
    const int64_t nblocks = ((ntm + kGM - 1) / kGM) * ((ntn + kGN - 1) / kGN);
    return (nblocks + kXcds - 1) / kXcds * kXcds * kGM * kGN;
}

// Waves kWN (n) x 2 (m); each wave owns 32 kNB outputs x 64 tokens (kNB x 2
// blocks of 32 x 32 accumulators). A stage moves 256 + 128 rows of 64 bytes
// into LDS (kAL + kBL 16-byte pieces per thread, issued before the current
// stage's matrix work): straight from global memory into LDS when K is a
// multiple of kPK, else through registers with the last stage's missing
// pieces masked (KTAIL). K and N must be multiples of 8.
template <class Out, bool KTAIL>
__global__ __launch_bounds__(kGT) void mfma_kernel(const uint16_t* __restrict__ x, Weights wt,
                                                   int64_t M, int N, int K, int ntn, int64_t ntm,
                                                   Out out) {
    __shared__ Lds sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave % kWN, wm = wave / kWN;
    // this workgroup's tiles: group (block) b of its domain, place w in it;
    // places outside the tile grid end here, before any barrier
    int64_t tn, tm;
    {
        const int64_t id = blockIdx.x, xcd = id % kXcds, local = id / kXcds;
        const int64_t nbm = (ntm + kGM - 1) / kGM, nbn = (ntn + kGN - 1) / kGN;
        const int64_t b = (local / (kGM * kGN)) * kXcds + xcd;
        const int w = (int)(local % (kGM * kGN));
        if (b >= nbm * nbn) return;
        tm = (b % nbm) * kGM + w % kGM;
        tn = (b / nbm) * kGN + w / kGM;
        if (tm >= ntm || tn >= ntn) return;
    }
    const int n0 = (int)tn * kPN;
    const int64_t m0 = tm * kPM;

    f32x16 acc[kNB][kMB];
#pragma unroll
    for (int i = 0; i < kNB; ++i)
#pragma unroll
        for (int j = 0; j < kMB; ++j) acc[i][j] = (f32x16){};
    const int nstages = (K + kPK - 1) / kPK;
    const int fr = lane & 31, fk = 8 * (lane >> 5);
    auto compute = [&](int buf) {
#pragma unroll
        for (int kk = 0; kk < kPK; kk += 16) {
            const int q = (kk + fk) >> 3;   // logical piece of the fragment
            bf16x8 af[kNB], bfr[kMB];
#pragma unroll
            for (int i = 0; i < kNB; ++i) {
                const int row = wn * (32 * kNB) + 32 * i + fr;
                af[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)&sm.a[buf][row][8 * (q ^ swz(row))]);
            }
#pragma unroll
            for (int j = 0; j < kMB; ++j) {
                const int row = wm * 64 + 32 * j + fr;
                bfr[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)&sm.b[buf][row][8 * (q ^ swz(row))]);
            }
#pragma unroll
            for (int i = 0; i < kNB; ++i)
#pragma unroll
                for (int j = 0; j < kMB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j],
                                                                        0, 0, 0);
        }
    };

    // Each thread's row pointers are fixed for the whole k loop; rows past M
    // or N read the last row instead (their results are never stored), so a
    // stage's loads are plain pointer + k, no bounds test.
    if constexpr (!KTAIL) {
        // Stages go from global memory straight into LDS (one 16-byte piece
        // per lane, a wave's 64 pieces landing on 16 consecutive 64-byte rows
        // in lane order): no staging registers, no LDS store instructions.
        // Lane l of wave w fills row 16 w + l / 4 (+ kRows j) at position
        // l % 4, which holds logical piece (l % 4) ^ swz(row) = (l % 4) ^ (l / 16),
        // so it loads that piece. Stage s + 1 is in flight while stage s
        // computes; the barrier at the end of a stage waits for it.
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        const int pr = 16 * wv + (lane >> 2), pq = 8 * ((lane & 3) ^ (lane >> 4));
        const uint16_t* wp[kAL];
        const uint16_t* xp[kBL];
#pragma unroll
        for (int j = 0; j < kAL; ++j) wp[j] = wt.row<uint16_t>(min(n0 + pr + kRows * j, N - 1), K) + pq;
#pragma unroll
        for (int j = 0; j < kBL; ++j) xp[j] = x + min(m0 + pr + kRows * j, M - 1) * K + pq;
        typedef __attribute__((address_space(3))) void* lds_ptr;
        auto load_stage = [&](int k0, int buf) {
#pragma unroll
            for (int j = 0; j < kAL; ++j)
                __builtin_amdgcn_global_load_lds((const void*)(wp[j] + k0),
                                                 (lds_ptr)&sm.a[buf][16 * wv + kRows * j][0], 16, 0, 0);
#pragma unroll
            for (int j = 0; j < kBL; ++j)
                __builtin_amdgcn_global_load_lds((const void*)(xp[j] + k0),
                                                 (lds_ptr)&sm.b[buf][16 * wv + kRows * j][0], 16, 0, 0);
        };
        load_stage(0, 0);
        __syncthreads();
        for (int s = 0; s < nstages; ++s) {
            if (s + 1 < nstages) load_stage((s + 1) * kPK, (s + 1) & 1);
            compute(s & 1);
            __syncthreads();
        }
    } else {
        // K not a multiple of kPK: register staging, the last stage's missing
        // pieces masked to zero (row r = tid / 4 + kRows j, piece tid % 4)
        const int pr = tid >> 2, pc = (tid & 3) * 8;
        const uint16_t* wp[kAL];
        const uint16_t* xp[kBL];
#pragma unroll
        for (int j = 0; j < kAL; ++j) wp[j] = wt.row<uint16_t>(min(n0 + pr + kRows * j, N - 1), K) + pc;
#pragma unroll
        for (int j = 0; j < kBL; ++j) xp[j] = x + min(m0 + pr + kRows * j, M - 1) * K + pc;
        u32x4 ra[kAL], rb[kBL];
        auto load_stage = [&](int k0) {
            const bool ok = k0 + pc < K;
#pragma unroll
            for (int j = 0; j < kAL; ++j)
                ra[j] = ok ? *(const u32x4*)(wp[j] + k0) : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < kBL; ++j)
                rb[j] = ok ? *(const u32x4*)(xp[j] + k0) : (u32x4){0u, 0u, 0u, 0u};
        };
        auto store_stage = [&](int buf) {
#pragma unroll
            for (int j = 0; j < kAL; ++j)
                *(u32x4*)&sm.a[buf][pr + kRows * j][8 * ((pc >> 3) ^ swz(pr + kRows * j))] = ra[j];
#pragma unroll
            for (int j = 0; j < kBL; ++j)
                *(u32x4*)&sm.b[buf][pr + kRows * j][8 * ((pc >> 3) ^ swz(pr + kRows * j))] = rb[j];
        };
        // the next stage's rows travel into registers while this stage computes
        load_stage(0);
        store_stage(0);
        __syncthreads();
        for (int s = 0; s < nstages; ++s) {
            const int buf = s & 1;
            if (s + 1 < nstages) load_stage((s + 1) * kPK);
            compute(buf);
            if (s + 1 < nstages) store_stage(buf ^ 1);
            __syncthreads();
        }
    }

    // The results go out through LDS, one half of the tokens at a time: the
    // waves that own tokens 64 p .. 64 p + 63 write them as bf16 rows
    // [token][output] after the output step (D register r of lane l is
    // output 8 (r / 4) + 4 (l / 32) + r % 4 of its block, token l % 32), then
    // every thread stores 16-byte pieces of whole rows.
    constexpr int ORow = kPN + 8;   // padded row (bf16): 528 bytes, 16-byte aligned
    static_assert(64 * ORow * 2 <= (int)sizeof(Lds), "output staging fits the stage buffers");
    uint16_t* ot = (uint16_t*)&sm;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        if (wm == p) {
#pragma unroll
            for (int j = 0; j < kMB; ++j)
#pragma unroll
                for (int i = 0; i < kNB; ++i)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int ml = 32 * j + (lane & 31);
                        const int nl = wn * (32 * kNB) + 32 * i + 8 * g + 4 * (lane >> 5);
                        const int n = n0 + nl;
                        const f32x16& a = acc[i][j];
                        float f[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) f[e] = n < N ? out.act(a[4 * g + e], n + e) : 0.f;
                        const bf16x2 lo = {(__bf16)f[0], (__bf16)f[1]};
                        const bf16x2 hi = {(__bf16)f[2], (__bf16)f[3]};
                        *(u32x2*)&ot[ml * ORow + nl] = (u32x2){__builtin_bit_cast(uint32_t, lo),
                                                               __builtin_bit_cast(uint32_t, hi)};
                    }
        }
        __syncthreads();
#pragma unroll
        for (int q = tid; q < 64 * (kPN / 8); q += kGT) {
            const int ml = q / (kPN / 8), pc2 = q % (kPN / 8);
            const int64_t m = m0 + 64 * p + ml;
            const int n = n0 + 8 * pc2;
            if (m < M && n < N) *(u32x4*)out.at(m, n) = *(const u32x4*)&ot[ml * ORow + 8 * pc2];
        }
        __syncthreads();
    }
}

// fp32: 64 x 64 outputs per workgroup, each thread 4 x 4, fp32 accumulation.
template <class Out>
__global__ __launch_bounds__(256) void f32_kernel(const float* __restrict__ x, Weights wt,
                                                  int64_t M, int N, int K, Out out) {
    constexpr int T = 64, KT = 16;
    __shared__ float xs[KT][T + 1];   // [k][m]
    __shared__ float ws[KT][T + 1];   // [k][n]
    const int tid = threadIdx.x, tm = tid & 15, tn = tid >> 4;
    const int64_t m0 = block_y() * T;
    if (m0 >= M) return;
    const int n0 = blockIdx.x * T;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += KT) {
        __syncthreads();
        for (int i = tid; i < T * KT; i += 256) {
            const int r = i / KT, k = i % KT;
            const int64_t m = m0 + r;
            const int n = n0 + r;
            xs[k][r] = (m < M && k0 + k < K) ? x[m * K + k0 + k] : 0.f;
            ws[k][r] = (n < N && k0 + k < K) ? wt.row<float>(n, K)[k0 + k] : 0.f;
        }
        __syncthreads();
#pragma unroll 4
        for (int k = 0; k < KT; ++k) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = xs[k][tm + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = ws[k][tn + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + tm + 16 * i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tn + 16 * j;
            if (n < N) *out.at(m, n) = out.act(acc[i][j], n);
        }
    }
}

// Launches C = out(x W^T) for M tokens, N outputs, K inputs.
template <class OutB, class OutF>
inline hipError_t launch(bool bf16, const void* x, Weights wt, int64_t M, int N, int K,
                         const OutB& ob, const OutF& of, hipStream_t st) {
    if (M == 0 || N == 0) return hipSuccess;
    if (bf16) {
        const int ntn = (N + kPN - 1) / kPN;
        const int64_t ntm = (M + kPM - 1) / kPM;
        const unsigned grid = (unsigned)mfma_grid(ntn, ntm);
        if (K % kPK)
            mfma_kernel<OutB, true><<<grid, kGT, 0, st>>>((const uint16_t*)x, wt, M, N, K, ntn,
                                                          ntm, ob);
        else
            mfma_kernel<OutB, false><<<grid, kGT, 0, st>>>((const uint16_t*)x, wt, M, N, K, ntn,
                                                           ntm, ob);
    } else {
        const dim3 grid = grid_split((unsigned)((N + 63) / 64), (M + 63) / 64);
        f32_kernel<OutF><<<grid, 256, 0, st>>>((const float*)x, wt, M, N, K, of);
    }
    return hipGetLastError();
}

}  // namespace gemm
}  // namespace lsh
