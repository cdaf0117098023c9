// lsh_combine.hip -- step 5: un-sort and combine the hash rounds.
//
// Method: twgreatdaily.com walkthrough, section "1 LSH Attention": with several
// rounds the attended set is the union of the rounds' sets. Each round's
// result o_r is normalised by its own partition function exp(lse_r); weighting
// it by exp(lse_r - logsumexp_r lse_r) gives one softmax over every (round,
// key) hit.
//
// One thread per (token, 8 features): the rounds' slots come through inv, the
// float32 rows of o_sorted are read as 16-byte vectors and the outputs are
// written with one vector store per thread.
#include "lsh_internal.h"

namespace lsh {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Stores 8 consecutive outputs with one vector store.
__device__ __forceinline__ void store8(float* p, const f32x4& a, const f32x4& b) {
    __builtin_nontemporal_store(a, (f32x4*)p);
    __builtin_nontemporal_store(b, (f32x4*)(p + 4));
}
__device__ __forceinline__ void store8(uint16_t* p, const f32x4& a, const f32x4& b) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 w;
    w.x = (uint32_t)f32_to_bf16(a.x) | ((uint32_t)f32_to_bf16(a.y) << 16);
    w.y = (uint32_t)f32_to_bf16(a.z) | ((uint32_t)f32_to_bf16(a.w) << 16);
    w.z = (uint32_t)f32_to_bf16(b.x) | ((uint32_t)f32_to_bf16(b.y) << 16);
    w.w = (uint32_t)f32_to_bf16(b.z) | ((uint32_t)f32_to_bf16(b.w) << 16);
    __builtin_nontemporal_store(w, (u32x4*)p);
}

// 8 consecutive per-round outputs of one row, as two float4. The rows are
// read exactly once, and the outputs are not read again here, so both go
// through the streaming (nontemporal) path and leave the caches alone.
template <bool HALF>
__device__ __forceinline__ void load8(const void* base, int64_t off, f32x4& a, f32x4& b) {
    if constexpr (HALF) {
        typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
        const f16x8 h = __builtin_nontemporal_load((const f16x8*)((const _Float16*)base + off));
        a = (f32x4){(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
        b = (f32x4){(float)h[4], (float)h[5], (float)h[6], (float)h[7]};
    } else {
        a = __builtin_nontemporal_load((const f32x4*)((const float*)base + off));
        b = __builtin_nontemporal_load((const f32x4*)((const float*)base + off + 4));
    }
}

// Staged form: per-round rows by sorted slot, reached through inv.
template <int D, typename T>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o_sorted,
                                                      const float* __restrict__ lse,
                                                      const int32_t* __restrict__ inv, Dims dm,
                                                      T* __restrict__ out, float* __restrict__ z) {
    constexpr int TPT = D / 8;   // threads per token, 8 features each
    constexpr int G = 8;         // rounds whose loads are issued together
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t tok = gid / TPT;
    const int q = (int)(gid - tok * TPT);
    if (tok >= dm.T) return;
    const int64_t L = dm.L;
    const int64_t bh = tok / L;
    const int64_t i = tok - bh * L;
    const int64_t seg0 = bh * dm.nh;
    // exp(l_r - Z) is evaluated as exp(l_r - max) / sum_r exp(l_r - max) with a
    // running max: forming Z = max + log(sum) first would round it to the spacing
    // of floats near |max|, which is 2^-7 when a round saw only the query itself
    // (l_r ~ -1e5).
    float mx = -INFINITY, sum = 0.f;
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    for (int r0 = 0; r0 < dm.nh; r0 += G) {
        const int n = min(G, dm.nh - r0);
        int64_t slot[G];
        float l[G];
        f32x4 o0[G], o1[G];
#pragma unroll
        for (int k = 0; k < G; ++k)
            if (k < n) slot[k] = (seg0 + r0 + k) * L + inv[(seg0 + r0 + k) * L + i];
#pragma unroll
        for (int k = 0; k < G; ++k)
            if (k < n) {
                l[k] = lse[slot[k]];
                load8<false>(o_sorted, slot[k] * D + 8 * q, o0[k], o1[k]);
            }
        float gmx = mx;
#pragma unroll
        for (int k = 0; k < G; ++k)
            if (k < n) gmx = fmaxf(gmx, l[k]);
        // a round with lse -inf (no key: separate queries and keys only)
        // weighs 0; while every round so far is such, take exponentials
        // against 0 instead of -inf
        const float gref = gmx == -INFINITY ? 0.f : gmx;
        const float rescale = expf(mx - gref);   // 0 on the first group (mx = -inf)
        sum *= rescale;
        a0 *= rescale;
        a1 *= rescale;
#pragma unroll
        for (int k = 0; k < G; ++k)
            if (k < n) {
                const float e = expf(l[k] - gref);
                sum += e;
                a0 += e * o0[k];
                a1 += e * o1[k];
            }
        mx = gmx;
    }
    // sum = 0: no round has a key, the output row is zero
    const float inv_sum = sum > 0.f ? 1.0f / sum : 0.f;
    store8(out + tok * D + 8 * q, a0 * inv_sum, a1 * inv_sum);
    if (z && q == 0) z[tok] = sum > 0.f ? mx + logf(sum) : -INFINITY;
}

// Fused form: the chunk kernel already stored every round's row of a token
// next to each other ([token][round][d], scaled fp16), so the un-sort is done
// and this pass reads one contiguous block per token. Each 64-byte group of
// 32 features also carries the round's log2-domain lse in its values' lowest
// mantissa bits: word j of the group holds bit j in its low half and bit
// 16 + j in its high half. The thread owning 16-byte piece q of a row has
// words j = 4 (q % 4) .. +3; the four threads of a quad together see one
// whole group, so two DPP swaps assemble the value. G rounds' loads are
// issued together (2, 4 or 8: the round count rounded up, at most 8), so few
// rounds do not load and weigh padding rows.
template <int D, typename T, int G>
__global__ __launch_bounds__(256) void combine_bypos_kernel(const _Float16* __restrict__ o_pos,
                                                            const uint32_t* __restrict__ vmax,
                                                            Dims dm, T* __restrict__ out,
                                                            float* __restrict__ z) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    constexpr int TPT = D / 8;   // threads per token, one 16-byte piece each
    // Blocks run from the last token back: the chunk pass finishes with the
    // last (batch, head) slices, whose rows are then still in the memory-side
    // cache when this pass starts.
    const int64_t gid = (int64_t)(gridDim.x - 1 - blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t tok = gid / TPT;
    const int q = (int)(gid - tok * TPT);
    if (tok >= dm.T) return;   // whole tokens, so whole quads, drop out together
    const u32x4* rows = (const u32x4*)o_pos + tok * dm.nh * TPT + q;   // round r: rows[r * TPT]
    const int sh = 4 * (q & 3);
    float mx = -INFINITY, sum = 0.f;
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    for (int r0 = 0; r0 < dm.nh; r0 += G) {
        const int n = min(G, dm.nh - r0);
        // past the last round the last row is read again and weighted 0
        u32x4 w[G];
#pragma unroll
        for (int k = 0; k < G; ++k)
            w[k] = __builtin_nontemporal_load(rows + min(r0 + k, dm.nh - 1) * TPT);
        float l[G];
        float gmx = mx;
#pragma unroll
        for (int k = 0; k < G; ++k) {
            uint32_t b = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) b |= (w[k][i] & 0x10001u) << (sh + i);
            b |= (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0xB1, 0xF, 0xF, false);   // quad [1,0,3,2]
            b |= (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0x4E, 0xF, 0xF, false);   // quad [2,3,0,1]
            l[k] = k < n ? __uint_as_float(b) : -INFINITY;
            gmx = fmaxf(gmx, l[k]);
        }
        // exp2(l - running max), the running max kept unrounded (a round that
        // saw only the query itself sits near -1e5 / ln 2); rounds with lse
        // -inf (no key: separate queries and keys only) weigh 0, and while
        // every round so far is such the reference is 0 instead of -inf
        const float gref = gmx == -INFINITY ? 0.f : gmx;
        const float rescale = __builtin_amdgcn_exp2f(mx - gref);   // 0 on the first group
        sum *= rescale;
        a0 *= rescale;
        a1 *= rescale;
#pragma unroll
        for (int k = 0; k < G; ++k) {
            const float e = __builtin_amdgcn_exp2f(l[k] - gref);   // 0 past the last round
            sum += e;
            const f32x4 lo = {(float)__builtin_bit_cast(_Float16, (uint16_t)w[k][0]),
                              (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k][0] >> 16)),
                              (float)__builtin_bit_cast(_Float16, (uint16_t)w[k][1]),
                              (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k][1] >> 16))};
            const f32x4 hi = {(float)__builtin_bit_cast(_Float16, (uint16_t)w[k][2]),
                              (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k][2] >> 16)),
                              (float)__builtin_bit_cast(_Float16, (uint16_t)w[k][3]),
                              (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k][3] >> 16))};
            a0 += e * lo;
            a1 += e * hi;
        }
        mx = gmx;
    }
    // the rows carry the power-of-two scale chosen from max|v|; sum = 0: no
    // round has a key, the output row is zero
    const float inv_sum = sum > 0.f ? 1.0f / (o_scale(*vmax) * sum) : 0.f;
    store8(out + tok * D + 8 * q, a0 * inv_sum, a1 * inv_sum);
    if (z && q == 0)
        z[tok] = sum > 0.f ? (mx + log2f(sum)) * 0.6931471805599453f : -INFINITY;   // natural log
}

template <typename T>
static void launch_t(const OSorted& o, const float* lse, const int32_t* inv, const Dims& d, T* out,
                     float* z, hipStream_t st) {
    const unsigned grid = (unsigned)((d.T * (d.d / 8) + 255) / 256);
    if (o.half) {
        const _Float16* op = (const _Float16*)o.ptr;
#define LSH_BYPOS(DD, GG) combine_bypos_kernel<DD, T, GG><<<grid, 256, 0, st>>>(op, o.vmax, d, out, z)
        const int g = d.nh <= 2 ? 2 : d.nh <= 4 ? 4 : 8;
        if (d.d == 64) {
            if (g == 2) LSH_BYPOS(64, 2);
            else if (g == 4) LSH_BYPOS(64, 4);
            else LSH_BYPOS(64, 8);
        } else {
            if (g == 2) LSH_BYPOS(128, 2);
            else if (g == 4) LSH_BYPOS(128, 4);
            else LSH_BYPOS(128, 8);
        }
#undef LSH_BYPOS
    } else {
        const float* op = (const float*)o.ptr;
        if (d.d == 64)
            combine_kernel<64, T><<<grid, 256, 0, st>>>(op, lse, inv, d, out, z);
        else
            combine_kernel<128, T><<<grid, 256, 0, st>>>(op, lse, inv, d, out, z);
    }
}

hipError_t launch_combine(const OSorted& o, const float* lse_sorted, const int32_t* inv,
                          const Dims& d, void* out, hipStream_t st, hipEvent_t* ev, int* nev,
                          const char** names, float* z) {
    if (d.dtype == LSH_BF16)
        launch_t<uint16_t>(o, lse_sorted, inv, d, (uint16_t*)out, z, st);
    else
        launch_t<float>(o, lse_sorted, inv, d, (float*)out, z, st);
    return mark(st, ev, nev, names, "combine");
}

}  // namespace lsh
