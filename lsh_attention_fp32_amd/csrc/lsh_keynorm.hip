// lsh_keynorm.hip -- inverse key norms for the key-normalisation variant.
//
// Method: walkthrough "1 LSH Attention" (the key side of a score is the unit
// vector of the shared query/key vector). rn[t] = 1 / |qk[t]| in float32, 0
// for the zero vector, one value per (batch, head, position). The entry
// points that own a workspace compute it once per call, so the attention and
// backward kernels read one float next to each position instead of summing
// the squares of every row they stage.
#include "lsh_internal.h"

namespace lsh {

namespace {

// D/8 consecutive lanes per token, 8 features each, summed across the group.
template <int D, typename T>
__global__ __launch_bounds__(256) void key_rnorm_kernel(const T* __restrict__ qk, Dims dm,
                                                        float* __restrict__ rn) {
    constexpr int LPT = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t tok = gid / LPT;
    const int part = (int)(gid % LPT);
    float ss = 0.f;
    if (tok < dm.T) {
        const T* row = qk + tok * D + part * 8;
        const auto a = IO<T>::load4(row, 0);
        const auto b = IO<T>::load4(row, 4);
        ss = a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
        ss += b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
    }
#pragma unroll
    for (int o = 1; o < LPT; o <<= 1) ss += __shfl_xor(ss, o);   // whole groups share a token
    if (tok < dm.T && part == 0) rn[tok] = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
}

template <int D, typename T>
void launch_t(const void* qk, const Dims& d, float* rn, hipStream_t st) {
    const int64_t threads = d.T * (D / 8);
    key_rnorm_kernel<D, T><<<(unsigned)((threads + 255) / 256), 256, 0, st>>>((const T*)qk, d, rn);
}

}  // namespace

hipError_t launch_key_rnorm(const void* qk, const Dims& d, float* rn, hipStream_t st) {
    if (d.T == 0) return hipSuccess;
    if (d.dtype == LSH_BF16)
        d.d == 64 ? launch_t<64, uint16_t>(qk, d, rn, st) : launch_t<128, uint16_t>(qk, d, rn, st);
    else
        d.d == 64 ? launch_t<64, float>(qk, d, rn, st) : launch_t<128, float>(qk, d, rn, st);
    return hipGetLastError();
}

}  // namespace lsh
