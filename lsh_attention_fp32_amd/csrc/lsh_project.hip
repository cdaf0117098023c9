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
// One product over the concatenated outputs: out[m][n] = sum_k x[m][k] W[n][k],
// m = b*L + l, n < H*d from w_qk and n >= H*d from w_v; the store splits heads
// on the fly (8 consecutive outputs of a token are 16 contiguous bytes of one
// head's row in [B,H,L,d]).
#include "lsh_gemm.h"

namespace lsh {

namespace {

// Where output n of token m goes: qk or v, row (b, h, l), feature e.
template <typename T>
struct HeadSplit {
    T* qk;
    T* v;
    int64_t L;
    int H, d, hd;
    __device__ __forceinline__ float act(float a, int) const { return a; }
    __device__ __forceinline__ T* at(int64_t m, int n) const {
        T* base = qk;
        if (n >= hd) {
            base = v;
            n -= hd;
        }
        const int h = n / d, e = n - h * d;
        const int64_t b = m / L, l = m - b * L;
        return base + (((b * H + h) * L + l) * d + e);
    }
};

}  // namespace

hipError_t launch_project(const void* x, const void* w_qk, const void* w_v, const Dims& d,
                          int d_model, void* qk, void* v, hipStream_t st) {
    const int64_t M = (int64_t)d.B * d.L;
    const int hd = d.H * d.d;
    const gemm::Weights wt{w_qk, w_v, hd};
    const HeadSplit<uint16_t> ob{(uint16_t*)qk, (uint16_t*)v, d.L, d.H, d.d, hd};
    const HeadSplit<float> of{(float*)qk, (float*)v, d.L, d.H, d.d, hd};
    return gemm::launch(d.dtype == LSH_BF16, x, wt, M, 2 * hd, d_model, ob, of, st);
}

}  // namespace lsh
