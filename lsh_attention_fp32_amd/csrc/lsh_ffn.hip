// lsh_ffn.hip -- the chunked feed-forward.
//
// Method: twgreatdaily.com walkthrough, sections "3 分塊" (the feed-forward's
// positions are independent, so the sequence is cut into chunks computed one
// after another, bounding the wide intermediate) and the list of problems
// (the feed-forward's inner width exceeds the model width); ai-scholar.tech
// summary, section "Reformerを用いた結果" (d_model 1024, d_ff 4096). Reading:
// the Transformer's position-wise feed-forward with a ReLU between two linear
// maps and a bias after each (NULL biases are zero), weights output-major:
//   out[m] = relu(x[m] W1^T + b1) W2^T + b2.
//
// Per chunk of rows: one product into the chunk's intermediate (bias and ReLU
// applied before the rounding to the I/O dtype), one product out of it. The
// intermediate of a chunk is rows * d_ff elements of workspace; with chunks of
// a few thousand rows it stays in the last-level cache between the two
// products.
#include <algorithm>

#include "lsh_gemm.h"

namespace lsh {

namespace {

// Row-major output [M][ldc] with a bias per output and an optional ReLU.
template <typename T, bool RELU>
struct RowOut {
    T* c;
    int64_t ldc;
    const T* bias;
    __device__ __forceinline__ float act(float a, int n) const {
        const float v = bias ? a + IO<T>::load(bias, n) : a;
        return RELU ? fmaxf(v, 0.f) : v;
    }
    __device__ __forceinline__ T* at(int64_t m, int n) const { return c + m * ldc + n; }
};

template <bool RELU>
hipError_t product(bool bf16, const void* x, const void* w, const void* bias, int64_t M, int N,
                   int K, void* c, hipStream_t st) {
    const gemm::Weights wt{w, w, N};
    const RowOut<uint16_t, RELU> ob{(uint16_t*)c, N, (const uint16_t*)bias};
    const RowOut<float, RELU> of{(float*)c, N, (const float*)bias};
    return gemm::launch(bf16, x, wt, M, N, K, ob, of, st);
}

}  // namespace

hipError_t launch_ffn(const void* x, const void* w1, const void* b1, const void* w2,
                      const void* b2, int64_t rows, int d_model, int d_ff, int chunk_rows,
                      bool bf16, void* out, void* inter, hipStream_t st) {
    const size_t e = bf16 ? 2 : 4;
    for (int64_t r0 = 0; r0 < rows; r0 += chunk_rows) {
        const int64_t n = std::min<int64_t>(chunk_rows, rows - r0);
        const char* xc = (const char*)x + r0 * d_model * e;
        char* oc = (char*)out + r0 * d_model * e;
        hipError_t err = product<true>(bf16, xc, w1, b1, n, d_ff, d_model, inter, st);
        if (err == hipSuccess) err = product<false>(bf16, inter, w2, b2, n, d_model, d_ff, oc, st);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace lsh
