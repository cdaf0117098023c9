// lsh_combine.hip -- step 5: un-sort and combine the hash rounds.
//
// Method: twgreatdaily.com walkthrough, section "1 LSH Attention": with several
// rounds the attended set is the union of the rounds' sets. Each round's
// result o_r is normalised by its own partition function exp(lse_r); weighting
// it by exp(lse_r - logsumexp_r lse_r) gives one softmax over every (round,
// key) hit.
//
// One thread per (token, 4 features): the rounds' slots come through inv, the
// float32 rows of o_sorted are read as 16-byte vectors.
#include "lsh_internal.h"

namespace lsh {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D, typename T>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o_sorted,
                                                      const float* __restrict__ lse,
                                                      const int32_t* __restrict__ inv, Dims dm,
                                                      T* __restrict__ out) {
    constexpr int TPT = D / 4;   // threads per token
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t tok = gid / TPT;
    const int q = (int)(gid - tok * TPT);
    if (tok >= dm.T) return;
    const int64_t L = dm.L;
    const int64_t bh = tok / L;
    const int64_t i = tok - bh * L;
    const int64_t seg0 = bh * dm.nh;
    float mx = -INFINITY;
    for (int r = 0; r < dm.nh; ++r) {
        const int64_t row = (seg0 + r) * L;
        mx = fmaxf(mx, lse[row + inv[row + i]]);
    }
    // exp(l_r - Z) is evaluated as exp(l_r - max) / sum_r exp(l_r - max): forming
    // Z = max + log(sum) first would round it to the spacing of floats near |max|,
    // which is 2^-7 when a round saw only the query itself (l_r ~ -1e5).
    float sum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < dm.nh; ++r) {
        const int64_t row = (seg0 + r) * L;
        const int64_t s = inv[row + i];
        const float e = expf(lse[row + s] - mx);
        const f32x4 o = *(const f32x4*)(o_sorted + (row + s) * D + 4 * q);
        sum += e;
        acc += e * o;
    }
    const float inv_sum = 1.0f / sum;
#pragma unroll
    for (int e = 0; e < 4; ++e) IO<T>::store(out, tok * D + 4 * q + e, acc[e] * inv_sum);
}

template <typename T>
static void launch_t(const float* o, const float* lse, const int32_t* inv, const Dims& d, T* out,
                     hipStream_t st) {
    const int64_t threads = d.T * (d.d / 4);
    const unsigned grid = (unsigned)((threads + 255) / 256);
    if (d.d == 64)
        combine_kernel<64, T><<<grid, 256, 0, st>>>(o, lse, inv, d, out);
    else
        combine_kernel<128, T><<<grid, 256, 0, st>>>(o, lse, inv, d, out);
}

hipError_t launch_combine(const float* o_sorted, const float* lse_sorted, const int32_t* inv,
                          const Dims& d, void* out, hipStream_t st, hipEvent_t* ev, int* nev,
                          const char** names) {
    if (d.dtype == LSH_BF16)
        launch_t(o_sorted, lse_sorted, inv, d, (uint16_t*)out, st);
    else
        launch_t(o_sorted, lse_sorted, inv, d, (float*)out, st);
    return mark(st, ev, nev, names, "combine");
}

}  // namespace lsh
