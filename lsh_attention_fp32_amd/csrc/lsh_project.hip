// lsh_project.hip -- the shared query/key and the value input projections.
//
// Method: ultralytics.com glossary, section "Atenção LSH" (queries and keys
// come from one shared projection); ai-scholar.tech summary, section
// "Reformerを用いた結果" (model width 1024 split over 8 heads). Reading: two
// bias-free linear maps of the token vectors, weights stored output-major
// (w[n][k] for output n, input k, the layout of a linear layer's weight), head
// h taking outputs h*d .. h*d + d - 1:
//   qk[b,h,l,e] = sum_k x[b,l,k] w_qk[h*d+e][k],  v likewise with w_v.
//
// One GEMM over the concatenated outputs: out[m][n] = sum_k x[m][k] W[n][k],
// m = b*L + l, n < H*d from w_qk and n >= H*d from w_v. It runs as
// out^T = W x^T on v_mfma_f32_32x32x16_bf16 (A = weight rows, B = token rows:
// both are read along k, so every operand fragment is one 16-byte piece of a
// row), and the store splits heads on the fly: a lane holds four consecutive
// outputs of one token, which land as 8 contiguous bytes of [B,H,L,d].
#include "lsh_internal.h"

namespace lsh {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPN = 256;        // outputs (n) per workgroup
constexpr int kPM = 128;        // tokens (m) per workgroup
constexpr int kPK = 32;         // k per LDS stage
constexpr int kPRow = kPK + 8;  // padded LDS row (bf16): 80 bytes, rows 20 banks apart
constexpr int kXcds = 8;        // L2 domains the dispatcher deals workgroups over

struct ProjectLds {
    uint16_t a[2][kPN][kPRow];   // weight rows
    uint16_t b[2][kPM][kPRow];   // token rows
};

// Where output n of token m goes: qk or v, row (b, h, l), feature e.
struct OutMap {
    uint16_t* qk;
    uint16_t* v;
    int64_t L;
    int H, d, hd;
    __device__ __forceinline__ uint16_t* at(int64_t m, int n) const {
        uint16_t* base = qk;
        if (n >= hd) {
            base = v;
            n -= hd;
        }
        const int h = n / d, e = n - h * d;
        const int64_t b = m / L, l = m - b * L;
        return base + (((b * H + h) * L + l) * d + e);
    }
};

// Waves 2 (n) x 2 (m); each wave owns 128 outputs x 64 tokens = 4 x 2 blocks
// of 32 x 32 accumulators. A stage moves 256 + 128 rows of 64 bytes from HBM
// into LDS (six 16-byte loads per thread, issued before the current stage's
// matrix work and stored after it).
__global__ __launch_bounds__(256) void project_mfma_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wqk,
                                                           const uint16_t* __restrict__ wv,
                                                           int64_t M, int N, int K, int ntn,
                                                           int64_t ntm, OutMap out) {
    __shared__ ProjectLds sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    // Workgroups are dealt round-robin over the L2 domains, so the linear id
    // is remapped: the ids that share a domain take one token tile through
    // every output tile in turn, and its token rows come from HBM once.
    int64_t tn, tm;
    {
        const int64_t id = blockIdx.x, total = (int64_t)ntn * ntm;
        const int64_t full = total / ((int64_t)kXcds * ntn) * ((int64_t)kXcds * ntn);
        if (id < full) {
            const int64_t xcd = id % kXcds, j = id / kXcds;
            tn = j % ntn;
            tm = (j / ntn) * kXcds + xcd;
        } else {   // the tail that does not fill every domain: plain order
            tn = (id - full) % ntn;
            tm = full / ntn + (id - full) / ntn;
        }
    }
    const int n0 = (int)tn * kPN;
    const int64_t m0 = tm * kPM;
    const int hd = N / 2;

    // global -> register staging: row r = tid / 4 + 64 j, piece tid % 4
    const int pr = tid >> 2, pc = (tid & 3) * 8;
    u32x4 ra[4], rb[2];
    auto load_stage = [&](int k0) {
        const int k = k0 + pc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + pr + 64 * j;
            ra[j] = (u32x4){0u, 0u, 0u, 0u};
            if (n < N && k < K) {
                const uint16_t* w = n < hd ? wqk + (int64_t)n * K : wv + (int64_t)(n - hd) * K;
                ra[j] = *(const u32x4*)(w + k);
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t m = m0 + pr + 64 * j;
            rb[j] = (u32x4){0u, 0u, 0u, 0u};
            if (m < M && k < K) rb[j] = *(const u32x4*)(x + m * K + k);
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) *(u32x4*)&sm.a[buf][pr + 64 * j][pc] = ra[j];
#pragma unroll
        for (int j = 0; j < 2; ++j) *(u32x4*)&sm.b[buf][pr + 64 * j][pc] = rb[j];
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16){};

    const int nstages = (K + kPK - 1) / kPK;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    const int fr = lane & 31, fk = 8 * (lane >> 5);
    for (int s = 0; s < nstages; ++s) {
        const int buf = s & 1;
        if (s + 1 < nstages) load_stage((s + 1) * kPK);
#pragma unroll
        for (int kk = 0; kk < kPK; kk += 16) {
            bf16x8 af[4], bfr[2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = __builtin_bit_cast(
                    bf16x8, *(const u32x4*)&sm.a[buf][wn * 128 + 32 * i + fr][kk + fk]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bfr[j] = __builtin_bit_cast(
                    bf16x8, *(const u32x4*)&sm.b[buf][wm * 64 + 32 * j + fr][kk + fk]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j],
                                                                        0, 0, 0);
        }
        if (s + 1 < nstages) store_stage(buf ^ 1);
        __syncthreads();
    }

    // The results go out through LDS, one half of the tokens at a time: the
    // waves that own tokens 64 p .. 64 p + 63 write them as bf16 rows
    // [token][output] (D register r of lane l is output 8 (r / 4) + 4 (l / 32)
    // + r % 4 of its block, token l % 32), then every thread stores 16-byte
    // pieces of whole rows, each piece 8 consecutive features of one head.
    constexpr int ORow = kPN + 8;   // padded row (bf16): 528 bytes, 16-byte aligned
    static_assert(64 * ORow * 2 <= (int)sizeof(ProjectLds), "output staging fits the stage buffers");
    uint16_t* ot = (uint16_t*)&sm;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        if (wm == p) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int ml = 32 * j + (lane & 31);
                        const int nl = wn * 128 + 32 * i + 8 * g + 4 * (lane >> 5);
                        const f32x16& a = acc[i][j];
                        *(u32x2*)&ot[ml * ORow + nl] =
                            (u32x2){(uint32_t)f32_to_bf16(a[4 * g]) |
                                        ((uint32_t)f32_to_bf16(a[4 * g + 1]) << 16),
                                    (uint32_t)f32_to_bf16(a[4 * g + 2]) |
                                        ((uint32_t)f32_to_bf16(a[4 * g + 3]) << 16)};
                    }
        }
        __syncthreads();
#pragma unroll
        for (int q = tid; q < 64 * (kPN / 8); q += 256) {
            const int ml = q / (kPN / 8), pc = q % (kPN / 8);
            const int64_t m = m0 + 64 * p + ml;
            const int n = n0 + 8 * pc;
            if (m < M && n < N) *(u32x4*)out.at(m, n) = *(const u32x4*)&ot[ml * ORow + 8 * pc];
        }
        __syncthreads();
    }
}

// fp32 inputs: a plain LDS-tiled kernel, 64 x 64 outputs per workgroup, each
// thread 4 x 4, fp32 accumulation.
__global__ __launch_bounds__(256) void project_f32_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ wqk,
                                                          const float* __restrict__ wv,
                                                          int64_t M, int N, int K, float* qk,
                                                          float* v, int64_t L, int H, int d) {
    constexpr int T = 64, KT = 16;
    __shared__ float xs[KT][T + 1];   // [k][m]
    __shared__ float ws[KT][T + 1];   // [k][n]
    const int tid = threadIdx.x, tm = tid & 15, tn = tid >> 4;
    const int64_t m0 = (int64_t)blockIdx.y * T;
    const int n0 = blockIdx.x * T;
    const int hd = N / 2;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += KT) {
        __syncthreads();
        for (int i = tid; i < T * KT; i += 256) {
            const int r = i / KT, k = i % KT;
            const int64_t m = m0 + r;
            const int n = n0 + r;
            xs[k][r] = (m < M && k0 + k < K) ? x[m * K + k0 + k] : 0.f;
            float wval = 0.f;
            if (n < N && k0 + k < K)
                wval = n < hd ? wqk[(int64_t)n * K + k0 + k] : wv[(int64_t)(n - hd) * K + k0 + k];
            ws[k][r] = wval;
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
        const int64_t b = m / L, l = m - b * L;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int n = n0 + tn + 16 * j;
            if (n >= N) continue;
            float* base = qk;
            if (n >= hd) {
                base = v;
                n -= hd;
            }
            const int h = n / d, e = n - h * d;
            base[((b * H + h) * L + l) * d + e] = acc[i][j];
        }
    }
}

}  // namespace

hipError_t launch_project(const void* x, const void* w_qk, const void* w_v, const Dims& d,
                          int d_model, void* qk, void* v, hipStream_t st) {
    const int64_t M = (int64_t)d.B * d.L;
    const int N = 2 * d.H * d.d;
    if (M == 0) return hipSuccess;
    if (d.dtype == LSH_BF16) {
        const int ntn = (N + kPN - 1) / kPN;
        const int64_t ntm = (M + kPM - 1) / kPM;
        const OutMap om{(uint16_t*)qk, (uint16_t*)v, d.L, d.H, d.d, d.H * d.d};
        project_mfma_kernel<<<(unsigned)(ntn * ntm), 256, 0, st>>>(
            (const uint16_t*)x, (const uint16_t*)w_qk, (const uint16_t*)w_v, M, N, d_model, ntn,
            ntm, om);
    } else {
        const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
        project_f32_kernel<<<grid, 256, 0, st>>>((const float*)x, (const float*)w_qk,
                                                 (const float*)w_v, M, N, d_model, (float*)qk,
                                                 (float*)v, d.L, d.H, d.d);
    }
    return hipGetLastError();
}

}  // namespace lsh
