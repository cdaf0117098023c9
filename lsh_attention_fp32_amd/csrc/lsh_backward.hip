// lsh_backward.hip -- gradients of the forward with respect to qk and v.
//
// Method: the forward (walkthrough "1 LSH Attention"; glossary "Atenção
// LSH") gives each position one softmax over every (round, key) hit of its
// rounds' windows, so with Z_i the log of the total partition function
// (logsumexp over rounds of each round's lse), P_i(r,j) = exp(s_ij - Z_i) and
// out_i = sum_{r,j} P_i(r,j) v_j. For an output gradient g, with
// D_i = g_i . out_i and the scale 1/sqrt(d) (scholar "Transformerの問題点とは"):
//   dv_j += P g_i,   dS = P (g_i . v_j - D_i),
//   dq_i += dS x_j / sqrt(d),   dk_j += dS x_i / sqrt(d),   dqk = dq + dk
// (queries and keys are the same vectors). The hash and the sort are
// piecewise constant and carry no gradient; the backward re-reads the sorted
// order and bucket ids the forward saved, and Z.
//
// Four launches, no atomics, deterministic:
//   bwd_dot     D_i per token;
//   bwd_dq      per (round, chunk, 64 query slots): the window's keys pass
//               through LDS 32 at a time; dq of the round is written to a row
//               [B,H,L,n_hashes,d] (float32) at the query's position;
//   bwd_dkv     per (round, chunk, 64 key slots): the queries whose window
//               holds the key (this chunk and the next) pass through LDS 32 at
//               a time; dk is added to the key position's row of the round
//               (each row is owned by one quad of lanes), dv is written to a
//               second set of rows;
//   bwd_reduce  sums each position's rows over the rounds into dqk and dv.
// Four lanes share a query (or key), each holding a quarter of its features;
// dot products are summed across the quad.
//
// A position that sees only itself in every round (under causality, the
// first of its bucket in each round) has Z = s_ii - penalty + log(n_hashes),
// and each round's self pair weighs exactly 1 / n_hashes. In float32 the
// score and Z near -1e5 keep only about 7 fractional bits, so exp(s - Z)
// would be off by up to 1 %; such positions are recognised by Z below half
// the penalty (a key that counts lifts Z far above that) and get the exact
// weight.
#include "lsh_internal.h"

namespace lsh {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// Position and bucket id of sorted slot t of a segment.
template <bool PACKED>
__device__ __forceinline__ void read_key(const int32_t* perm, const int32_t* bkt, int64_t t,
                                         int32_t& pos, int32_t& b) {
    const int32_t k = perm[t];
    if constexpr (PACKED) {
        pos = (int32_t)((uint32_t)k & kPackPosMask);
        b = (int32_t)((uint32_t)k >> kPackPosBits);
    } else {
        pos = k;
        b = bkt[k];
    }
}

template <int QD, typename T>
__device__ __forceinline__ void load_quarter(const T* row, int part, float (&r)[QD]) {
#pragma unroll
    for (int e = 0; e < QD; e += 4) {
        const f32x4 a = IO<T>::load4(row, part * QD + e);
        r[e] = a.x;
        r[e + 1] = a.y;
        r[e + 2] = a.z;
        r[e + 3] = a.w;
    }
}

// Weight of a valid (query, key) pair: exp(s - Z) in the exp2 domain, or
// 1 / n_hashes for the self pair of a position that sees only itself.
__device__ __forceinline__ float pair_weight(bool ok, bool self, float s2, float z2,
                                             bool self_only, float inv_nh) {
    if (!ok) return 0.f;
    if (self_only) return self ? inv_nh : 0.f;
    return __builtin_amdgcn_exp2f(s2 - z2);
}

__device__ __forceinline__ float quad_sum(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    return x;
}

// D_i = g_i . out_i, four lanes per token.
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_dot_kernel(const T* __restrict__ g,
                                                      const T* __restrict__ out, Dims dm,
                                                      float* __restrict__ Dv) {
    constexpr int QD = D / 4;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t tok = gid >> 2;
    const int part = (int)(gid & 3);
    if (tok >= dm.T) return;   // whole quads drop out together
    float a[QD], b[QD];
    load_quarter<QD>(g + tok * D, part, a);
    load_quarter<QD>(out + tok * D, part, b);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < QD; ++e) s = fmaf(a[e], b[e], s);
    s = quad_sum(s);
    if (part == 0) Dv[tok] = s;
}

template <int D, typename T, bool PACKED>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const T* __restrict__ qk,
                                                     const T* __restrict__ v,
                                                     const T* __restrict__ g,
                                                     const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ buckets,
                                                     const float* __restrict__ z,
                                                     const float* __restrict__ Dv, Dims dm,
                                                     int nqb, float* __restrict__ dx_r) {
    constexpr int QD = D / 4, KB = 32, KS = D + 4;
    __shared__ __attribute__((aligned(16))) float ks[KB][KS];
    __shared__ __attribute__((aligned(16))) float vs[KB][KS];
    __shared__ int32_t kpos[KB], kbkt[KB];
    const int64_t seg = blockIdx.y;
    const int64_t c = blockIdx.x / nqb;
    const int qb = (int)(blockIdx.x - c * nqb);
    const int tid = threadIdx.x, ql = tid >> 2, part = tid & 3;
    const int64_t L = dm.L, m = dm.m;
    const int64_t bh = seg / dm.nh;
    const int r = (int)(seg - bh * dm.nh);
    const int32_t* P = perm + seg * L;
    const int32_t* Bk = buckets + seg * L;
    const T* X = qk + bh * L * D;
    const T* V = v + bh * L * D;
    const T* G = g + bh * L * D;
    const int64_t qoff = (int64_t)qb * 64 + ql;
    const bool qlive = qoff < m;
    const int64_t s = c * m + (qlive ? qoff : 0);
    int32_t qpos, qbkt;
    read_key<PACKED>(P, Bk, s, qpos, qbkt);
    float q[QD], gq[QD], dq[QD];
    load_quarter<QD>(X + (int64_t)qpos * D, part, q);
    load_quarter<QD>(G + (int64_t)qpos * D, part, gq);
#pragma unroll
    for (int e = 0; e < QD; ++e) dq[e] = 0.f;
    const float zq = z[bh * L + qpos];
    const float z2 = zq * kLog2e;
    const bool self_only = zq < -0.5f * kSelfPenalty;
    const float inv_nh = 1.0f / (float)dm.nh;
    const float Di = Dv[bh * L + qpos];
    const float c2 = kLog2e / sqrtf((float)D);
    const float pen2 = kSelfPenalty * kLog2e;
    const int64_t t0 = c > 0 ? (c - 1) * m : 0, t1 = (c + 1) * m;
    for (int64_t kb0 = t0; kb0 < t1; kb0 += KB) {
        const int nk = (int)min((int64_t)KB, t1 - kb0);
        __syncthreads();
        if (tid < KB) {
            int32_t p = -1, b = 0;
            if (tid < nk) read_key<PACKED>(P, Bk, kb0 + tid, p, b);
            kpos[tid] = p;
            kbkt[tid] = b;
        }
        __syncthreads();
        for (int i = tid; i < KB * (D / 4); i += 256) {
            const int j = i / (D / 4), k = 4 * (i % (D / 4));
            const int32_t p = kpos[j];
            f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
            if (p >= 0) {
                a = IO<T>::load4(X, (int64_t)p * D + k);
                b = IO<T>::load4(V, (int64_t)p * D + k);
            }
            *(f32x4*)&ks[j][k] = a;
            *(f32x4*)&vs[j][k] = b;
        }
        __syncthreads();
        for (int j = 0; j < nk; ++j) {
            float dot = 0.f, gv = 0.f;
#pragma unroll
            for (int e = 0; e < QD; e += 4) {
                const f32x4 kk = *(const f32x4*)&ks[j][part * QD + e];
                const f32x4 vv = *(const f32x4*)&vs[j][part * QD + e];
                dot = fmaf(q[e], kk.x, fmaf(q[e + 1], kk.y, fmaf(q[e + 2], kk.z, fmaf(q[e + 3], kk.w, dot))));
                gv = fmaf(gq[e], vv.x, fmaf(gq[e + 1], vv.y, fmaf(gq[e + 2], vv.z, fmaf(gq[e + 3], vv.w, gv))));
            }
            dot = quad_sum(dot);
            gv = quad_sum(gv);
            const int32_t kp = kpos[j];
            const bool ok = kbkt[j] == qbkt && (!dm.causal || kp <= qpos);
            const float s2 = dot * c2 - (kp == qpos ? pen2 : 0.f);
            const float p = pair_weight(ok, kp == qpos, s2, z2, self_only, inv_nh);
            const float ds = p * (gv - Di);
#pragma unroll
            for (int e = 0; e < QD; e += 4) {
                const f32x4 kk = *(const f32x4*)&ks[j][part * QD + e];
                dq[e] = fmaf(ds, kk.x, dq[e]);
                dq[e + 1] = fmaf(ds, kk.y, dq[e + 1]);
                dq[e + 2] = fmaf(ds, kk.z, dq[e + 2]);
                dq[e + 3] = fmaf(ds, kk.w, dq[e + 3]);
            }
        }
    }
    if (!qlive) return;
    const float scale = 1.0f / sqrtf((float)D);
    float* row = dx_r + ((bh * L + qpos) * dm.nh + r) * D + part * QD;
#pragma unroll
    for (int e = 0; e < QD; e += 4)
        *(f32x4*)(row + e) = (f32x4){dq[e], dq[e + 1], dq[e + 2], dq[e + 3]} * scale;
}

template <int D, typename T, bool PACKED>
__global__ __launch_bounds__(256) void bwd_dkv_kernel(const T* __restrict__ qk,
                                                      const T* __restrict__ v,
                                                      const T* __restrict__ g,
                                                      const int32_t* __restrict__ perm,
                                                      const int32_t* __restrict__ buckets,
                                                      const float* __restrict__ z,
                                                      const float* __restrict__ Dv, Dims dm,
                                                      int nkb, float* __restrict__ dx_r,
                                                      float* __restrict__ dv_r) {
    constexpr int QD = D / 4, QB = 32, QS = D + 4;
    __shared__ __attribute__((aligned(16))) float qs[QB][QS];
    __shared__ __attribute__((aligned(16))) float gs[QB][QS];
    __shared__ int32_t qposs[QB], qbkts[QB];
    __shared__ float qz[QB], qD[QB];
    const int64_t seg = blockIdx.y;
    const int64_t c = blockIdx.x / nkb;
    const int kb = (int)(blockIdx.x - c * nkb);
    const int tid = threadIdx.x, kl = tid >> 2, part = tid & 3;
    const int64_t L = dm.L, m = dm.m;
    const int64_t bh = seg / dm.nh;
    const int r = (int)(seg - bh * dm.nh);
    const int32_t* P = perm + seg * L;
    const int32_t* Bk = buckets + seg * L;
    const T* X = qk + bh * L * D;
    const T* V = v + bh * L * D;
    const T* G = g + bh * L * D;
    const int64_t koff = (int64_t)kb * 64 + kl;
    const bool klive = koff < m;
    const int64_t t = c * m + (klive ? koff : 0);
    int32_t kpos, kbkt;
    read_key<PACKED>(P, Bk, t, kpos, kbkt);
    float k[QD], vk[QD], dk[QD], dv[QD];
    load_quarter<QD>(X + (int64_t)kpos * D, part, k);
    load_quarter<QD>(V + (int64_t)kpos * D, part, vk);
#pragma unroll
    for (int e = 0; e < QD; ++e) dk[e] = dv[e] = 0.f;
    const float c2 = kLog2e / sqrtf((float)D);
    const float pen2 = kSelfPenalty * kLog2e;
    const float inv_nh = 1.0f / (float)dm.nh;
    // queries whose window holds this key: this chunk and the next
    const int64_t s0 = c * m, s1 = min((c + 2) * m, L);
    for (int64_t qb0 = s0; qb0 < s1; qb0 += QB) {
        const int nq = (int)min((int64_t)QB, s1 - qb0);
        __syncthreads();
        if (tid < QB) {
            int32_t p = -1, b = 0;
            if (tid < nq) read_key<PACKED>(P, Bk, qb0 + tid, p, b);
            qposs[tid] = p;
            qbkts[tid] = b;
            qz[tid] = p >= 0 ? z[bh * L + p] : 0.f;
            qD[tid] = p >= 0 ? Dv[bh * L + p] : 0.f;
        }
        __syncthreads();
        for (int i = tid; i < QB * (D / 4); i += 256) {
            const int j = i / (D / 4), e = 4 * (i % (D / 4));
            const int32_t p = qposs[j];
            f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
            if (p >= 0) {
                a = IO<T>::load4(X, (int64_t)p * D + e);
                b = IO<T>::load4(G, (int64_t)p * D + e);
            }
            *(f32x4*)&qs[j][e] = a;
            *(f32x4*)&gs[j][e] = b;
        }
        __syncthreads();
        for (int j = 0; j < nq; ++j) {
            float dot = 0.f, gv = 0.f;
#pragma unroll
            for (int e = 0; e < QD; e += 4) {
                const f32x4 qq = *(const f32x4*)&qs[j][part * QD + e];
                const f32x4 gg = *(const f32x4*)&gs[j][part * QD + e];
                dot = fmaf(k[e], qq.x, fmaf(k[e + 1], qq.y, fmaf(k[e + 2], qq.z, fmaf(k[e + 3], qq.w, dot))));
                gv = fmaf(vk[e], gg.x, fmaf(vk[e + 1], gg.y, fmaf(vk[e + 2], gg.z, fmaf(vk[e + 3], gg.w, gv))));
            }
            dot = quad_sum(dot);
            gv = quad_sum(gv);
            const int32_t qp = qposs[j];
            // the key counts for this query: same bucket and, if causal, not later
            const bool ok = qbkts[j] == kbkt && (!dm.causal || kpos <= qp);
            const float s2 = dot * c2 - (kpos == qp ? pen2 : 0.f);
            const float zq = qz[j];
            const float p = pair_weight(ok, kpos == qp, s2, zq * kLog2e,
                                        zq < -0.5f * kSelfPenalty, inv_nh);
            const float ds = p * (gv - qD[j]);
#pragma unroll
            for (int e = 0; e < QD; e += 4) {
                const f32x4 qq = *(const f32x4*)&qs[j][part * QD + e];
                const f32x4 gg = *(const f32x4*)&gs[j][part * QD + e];
                dk[e] = fmaf(ds, qq.x, dk[e]);
                dk[e + 1] = fmaf(ds, qq.y, dk[e + 1]);
                dk[e + 2] = fmaf(ds, qq.z, dk[e + 2]);
                dk[e + 3] = fmaf(ds, qq.w, dk[e + 3]);
                dv[e] = fmaf(p, gg.x, dv[e]);
                dv[e + 1] = fmaf(p, gg.y, dv[e + 1]);
                dv[e + 2] = fmaf(p, gg.z, dv[e + 2]);
                dv[e + 3] = fmaf(p, gg.w, dv[e + 3]);
            }
        }
    }
    if (!klive) return;
    const float scale = 1.0f / sqrtf((float)D);
    const int64_t row = ((bh * L + kpos) * dm.nh + r) * D + part * QD;
#pragma unroll
    for (int e = 0; e < QD; e += 4) {
        f32x4* px = (f32x4*)(dx_r + row + e);
        *px = *px + (f32x4){dk[e], dk[e + 1], dk[e + 2], dk[e + 3]} * scale;
        *(f32x4*)(dv_r + row + e) = (f32x4){dv[e], dv[e + 1], dv[e + 2], dv[e + 3]};
    }
}

// dqk_i = sum_r dx_r[i], dv_i = sum_r dv_r[i]; one thread per (token, 4 features).
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float* __restrict__ dx_r,
                                                         const float* __restrict__ dv_r, Dims dm,
                                                         T* __restrict__ dqk, T* __restrict__ dv) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t tok = gid / (D / 4);
    const int e = 4 * (int)(gid - tok * (D / 4));
    if (tok >= dm.T) return;
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < dm.nh; ++r) {
        const int64_t row = (tok * dm.nh + r) * D + e;
        a += *(const f32x4*)(dx_r + row);
        b += *(const f32x4*)(dv_r + row);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        IO<T>::store(dqk, tok * D + e + i, a[i]);
        IO<T>::store(dv, tok * D + e + i, b[i]);
    }
}

template <int D, typename T, bool PACKED>
hipError_t launch_bwd_t(const BwdArgs& a, const Dims& d, hipStream_t st) {
    const T* qk = (const T*)a.qk;
    const T* v = (const T*)a.v;
    const T* g = (const T*)a.dout;
    const unsigned gq = (unsigned)((d.T * 4 + 255) / 256);
    bwd_dot_kernel<D, T><<<gq, 256, 0, st>>>(g, (const T*)a.out, d, a.Dv);
    const int nqb = (d.m + 63) / 64;
    const dim3 grid((unsigned)((int64_t)(d.L / d.m) * nqb), (unsigned)d.segs);
    bwd_dq_kernel<D, T, PACKED><<<grid, 256, 0, st>>>(qk, v, g, a.perm, a.buckets, a.z, a.Dv, d,
                                                      nqb, a.dx_r);
    bwd_dkv_kernel<D, T, PACKED><<<grid, 256, 0, st>>>(qk, v, g, a.perm, a.buckets, a.z, a.Dv, d,
                                                       nqb, a.dx_r, a.dv_r);
    const unsigned gr = (unsigned)((d.T * (D / 4) + 255) / 256);
    bwd_reduce_kernel<D, T><<<gr, 256, 0, st>>>(a.dx_r, a.dv_r, d, (T*)a.dqk, (T*)a.dv);
    return hipGetLastError();
}

template <typename T, bool PACKED>
hipError_t launch_bwd_d(const BwdArgs& a, const Dims& d, hipStream_t st) {
    return d.d == 64 ? launch_bwd_t<64, T, PACKED>(a, d, st) : launch_bwd_t<128, T, PACKED>(a, d, st);
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, const Dims& d, bool packed, hipStream_t st) {
    if (d.T == 0) return hipSuccess;
    if (d.dtype == LSH_BF16)
        return packed ? launch_bwd_d<uint16_t, true>(a, d, st) : launch_bwd_d<uint16_t, false>(a, d, st);
    return packed ? launch_bwd_d<float, true>(a, d, st) : launch_bwd_d<float, false>(a, d, st);
}

}  // namespace lsh
