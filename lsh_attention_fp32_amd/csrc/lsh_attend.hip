// lsh_attend.hip -- steps 3 and 4: gather into sorted order and chunked attention.
//
// Method: twgreatdaily.com walkthrough, section "1 LSH Attention" (keys are the
// queries, Q = K; only keys in the query's bucket take part, the others are
// masked out of a larger candidate set; chunks of m consecutive sorted items,
// each looking back exactly one chunk); ultralytics.com glossary, section
// "Atenção LSH" (own block and the previous block); ai-scholar.tech summary,
// section "Transformerの問題点とは" (scores scaled by 1/sqrt(d_k)).
//
// Window of sorted slot s in its round: slots of chunks c-1 and c, c = s / m
// (chunk 0 has no look-back, rounds never mix). Valid key: same bucket and,
// when causal, key position <= query position. A query's score against itself
// is lowered by kSelfPenalty, so it only counts when nothing else is valid.
#include "lsh_internal.h"

namespace lsh {

// Plain fp32 kernel: one thread per query slot, the window read through the
// cache, two passes (max, then exp-sum and weighted sum of V). Used for fp32
// inputs and any chunk length.
template <int D, typename T>
__global__ __launch_bounds__(128) void attend_valu_kernel(const T* __restrict__ qk,
                                                          const T* __restrict__ v,
                                                          const int32_t* __restrict__ buckets,
                                                          const int32_t* __restrict__ perm,
                                                          Dims dm, float* __restrict__ o_sorted,
                                                          float* __restrict__ lse_sorted) {
    const int64_t seg = blockIdx.y;
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= dm.L) return;
    const int64_t L = dm.L;
    const int64_t bh = seg / dm.nh;
    const int32_t* P = perm + seg * L;
    const int32_t* Bk = buckets + seg * L;
    const T* X = qk + bh * L * D;
    const T* V = v + bh * L * D;
    const int64_t i = P[s];
    const int bi = Bk[i];
    const int64_t c = s / dm.m;
    const int64_t t0 = c > 0 ? (c - 1) * dm.m : 0;
    const int64_t t1 = (c + 1) * dm.m;
    const float scale = 1.0f / sqrtf((float)D);
    const T* xi = X + i * D;

    float mx = -INFINITY;
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t j = P[t];
        if (Bk[j] != bi || (dm.causal && j > i)) continue;
        const T* xj = X + j * D;
        float dot = 0.f;
#pragma unroll 8
        for (int k = 0; k < D; ++k) dot = fmaf(IO<T>::load(xi, k), IO<T>::load(xj, k), dot);
        float sc = dot * scale;
        if (j == i) sc -= kSelfPenalty;
        mx = fmaxf(mx, sc);
    }
    float o[D];
#pragma unroll
    for (int k = 0; k < D; ++k) o[k] = 0.f;
    float sum = 0.f;
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t j = P[t];
        if (Bk[j] != bi || (dm.causal && j > i)) continue;
        const T* xj = X + j * D;
        float dot = 0.f;
#pragma unroll 8
        for (int k = 0; k < D; ++k) dot = fmaf(IO<T>::load(xi, k), IO<T>::load(xj, k), dot);
        float sc = dot * scale;
        if (j == i) sc -= kSelfPenalty;
        const float p = expf(sc - mx);
        sum += p;
        const T* vj = V + j * D;
#pragma unroll
        for (int k = 0; k < D; ++k) o[k] = fmaf(p, IO<T>::load(vj, k), o[k]);
    }
    const float inv_sum = 1.0f / sum;
    float* os = o_sorted + (seg * L + s) * D;
#pragma unroll
    for (int k = 0; k < D; ++k) os[k] = o[k] * inv_sum;
    lse_sorted[seg * L + s] = mx + logf(sum);
}

template <typename T>
static void launch_valu(const T* qk, const T* v, const int32_t* buckets, const int32_t* perm,
                        const Dims& d, float* o, float* lse, hipStream_t st) {
    dim3 grid((unsigned)((d.L + 127) / 128), (unsigned)d.segs);
    if (d.d == 64)
        attend_valu_kernel<64, T><<<grid, 128, 0, st>>>(qk, v, buckets, perm, d, o, lse);
    else
        attend_valu_kernel<128, T><<<grid, 128, 0, st>>>(qk, v, buckets, perm, d, o, lse);
}

hipError_t launch_attend(const void* qk, const void* v, const int32_t* buckets,
                         const int32_t* perm, const Dims& d, float* o_sorted, float* lse_sorted,
                         hipStream_t st, hipEvent_t* ev, int* nev, const char** names) {
    if (d.dtype == LSH_BF16)
        launch_valu((const uint16_t*)qk, (const uint16_t*)v, buckets, perm, d, o_sorted, lse_sorted,
                    st);
    else
        launch_valu((const float*)qk, (const float*)v, buckets, perm, d, o_sorted, lse_sorted, st);
    return mark(st, ev, nev, names, "attend_fp32");
}

}  // namespace lsh
