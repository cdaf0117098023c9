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
// (queries and keys are the same vectors). With key normalisation the score
// is s = (x_i . x_j) rn_j / sqrt(d), rn_j = 1 / |x_j|, so dq_i takes
// dS rn_j x_j and dk_j takes rn_j (dS x_i - rn_j^2 dS (x_i . x_j) x_j), both
// over sqrt(d); rn comes from a per-token pass before the kernels. The hash and the sort are
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
// With bf16 I/O and chunk 64 one matrix-core kernel (bwd_run) replaces the
// two middle passes and writes bf16 rows.
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

// The same dot for bf16 rows: D/8 lanes per token, one 16-byte nontemporal
// load of each row per lane (a wave's load covers whole rows, contiguous),
// fp32 products summed across the token's lanes.
template <int D>
__global__ __launch_bounds__(256) void bwd_dot_bf16_kernel(const uint16_t* __restrict__ g,
                                                           const uint16_t* __restrict__ out,
                                                           Dims dm, float* __restrict__ Dv) {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    constexpr int TPT = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t tok = gid / TPT;
    const int q = (int)(gid % TPT);
    if (tok >= dm.T) return;   // whole tokens drop out together
    const u32x4v a = __builtin_nontemporal_load((const u32x4v*)(g + tok * D) + q);
    const u32x4v b = __builtin_nontemporal_load((const u32x4v*)(out + tok * D) + q);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s = fmaf(__uint_as_float(a[i] << 16), __uint_as_float(b[i] << 16), s);
        s = fmaf(__uint_as_float(a[i] & 0xFFFF0000u), __uint_as_float(b[i] & 0xFFFF0000u), s);
    }
#pragma unroll
    for (int off = TPT / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (q == 0) Dv[tok] = s;
}

template <int D, typename T, bool PACKED>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const T* __restrict__ qk,
                                                     const T* __restrict__ v,
                                                     const T* __restrict__ g,
                                                     const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ buckets,
                                                     const float* __restrict__ z,
                                                     const float* __restrict__ Dv,
                                                     const float* __restrict__ rn, Dims dm,
                                                     int nqb, float* __restrict__ dx_r) {
    constexpr int QD = D / 4, KB = 32, KS = D + 4;
    __shared__ __attribute__((aligned(16))) float ks[KB][KS];
    __shared__ __attribute__((aligned(16))) float vs[KB][KS];
    __shared__ int32_t kpos[KB], kbkt[KB];
    __shared__ float krn[KB];   // 1 / |x_j| with key normalisation, else 1
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
            krn[tid] = (rn && p >= 0) ? rn[bh * L + p] : 1.f;
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
            const float s2 = dot * krn[j] * c2 - (kp == qpos ? pen2 : 0.f);
            const float p = pair_weight(ok, kp == qpos, s2, z2, self_only, inv_nh);
            const float ds = p * (gv - Di) * krn[j];
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
                                                      const float* __restrict__ Dv,
                                                      const float* __restrict__ rn, Dims dm,
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
    // the key's 1 / |x| and its sum of dS (x_i . x_j)
    const float krn = rn ? rn[bh * L + kpos] : 1.f;
    float sdd = 0.f;
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
            const float s2 = dot * krn * c2 - (kpos == qp ? pen2 : 0.f);
            const float zq = qz[j];
            const float p = pair_weight(ok, kpos == qp, s2, zq * kLog2e,
                                        zq < -0.5f * kSelfPenalty, inv_nh);
            const float ds = p * (gv - qD[j]);
            sdd = fmaf(ds, dot, sdd);
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
    if (rn) {
        const float pr = krn * krn * sdd;
#pragma unroll
        for (int e = 0; e < QD; ++e) dk[e] = krn * fmaf(-pr, k[e], dk[e]);
    }
    const float scale = 1.0f / sqrtf((float)D);
    const int64_t row = ((bh * L + kpos) * dm.nh + r) * D + part * QD;
#pragma unroll
    for (int e = 0; e < QD; e += 4) {
        f32x4* px = (f32x4*)(dx_r + row + e);
        *px = *px + (f32x4){dk[e], dk[e + 1], dk[e + 2], dk[e + 3]} * scale;
        *(f32x4*)(dv_r + row + e) = (f32x4){dv[e], dv[e + 1], dv[e + 2], dv[e + 3]};
    }
}

// Four consecutive values of a float32 per-round row.
__device__ __forceinline__ f32x4 load_row4(const float* p) { return *(const f32x4*)p; }

// dqk_i = sum_r dx_r[i], dv_i = sum_r dv_r[i]; one thread per (token, 4
// features), float32 rows of the plain passes.
template <int D, typename T, typename RowT>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const RowT* __restrict__ dx_r,
                                                         const RowT* __restrict__ dv_r, Dims dm,
                                                         T* __restrict__ dqk, T* __restrict__ dv) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t tok = gid / (D / 4);
    const int e = 4 * (int)(gid - tok * (D / 4));
    if (tok >= dm.T) return;
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < dm.nh; ++r) {
        const int64_t row = (tok * dm.nh + r) * D + e;
        a += load_row4(dx_r + row);
        b += load_row4(dv_r + row);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        IO<T>::store(dqk, tok * D + e + i, a[i]);
        IO<T>::store(dv, tok * D + e + i, b[i]);
    }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2 w = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, w);
}

// The same sum for the bf16 rows of the matrix-core pass and bf16 outputs:
// one thread per (token, 8 features), 16-byte nontemporal loads (the rows are
// read once), fp32 sums.
template <int D>
__global__ __launch_bounds__(256) void bwd_reduce_bf16_kernel(const uint16_t* __restrict__ dx_r,
                                                              const uint16_t* __restrict__ dv_r,
                                                              Dims dm, uint16_t* __restrict__ dqk,
                                                              uint16_t* __restrict__ dv) {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t tok = gid / (D / 8);
    const int e = 8 * (int)(gid - tok * (D / 8));
    if (tok >= dm.T) return;
    float a[8] = {}, b[8] = {};
#pragma unroll 4
    for (int r = 0; r < dm.nh; ++r) {
        const int64_t row = (tok * dm.nh + r) * D + e;
        const u32x4v wa = __builtin_nontemporal_load((const u32x4v*)(dx_r + row));
        const u32x4v wb = __builtin_nontemporal_load((const u32x4v*)(dv_r + row));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            a[2 * k] += __uint_as_float(wa[k] << 16);
            a[2 * k + 1] += __uint_as_float(wa[k] & 0xFFFF0000u);
            b[2 * k] += __uint_as_float(wb[k] << 16);
            b[2 * k + 1] += __uint_as_float(wb[k] & 0xFFFF0000u);
        }
    }
    u32x4v oa, ob;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        oa[k] = pack_bf16x2(a[2 * k], a[2 * k + 1]);
        ob[k] = pack_bf16x2(b[2 * k], b[2 * k + 1]);
    }
    *(u32x4v*)(dqk + tok * D + e) = oa;
    *(u32x4v*)(dv + tok * D + e) = ob;
}

// ---------------------------------------------------------------------------
// Matrix-core passes (bf16 I/O, chunk 64), v_mfma_f32_16x16x32_bf16 with fp32
// accumulation. Lane layout: A[m][k] in lane m%16 + 16*(k/8), element k%8;
// B[k][n] in lane n + 16*(k/8); D[m][n] in lane n + 16*(m/4), register m%4.
// A 16 x 16 score tile whose rows are the "other side" (keys in the query
// pass, queries in the key pass) takes row m from item
// 32 kb + 8 (m / 4) + 4 h + m % 4 of a 32-item block kb (h = 0, 1 the two
// tiles of the block): a lane then holds 8 consecutive items of the block,
// exactly the B-operand layout of the next product, so weights go from the
// score registers into the next matrix instruction without leaving the lane.
// The weights and dS are rounded to bf16 for those products.
constexpr int kBM = 64;   // chunk length of the matrix-core passes

template <int D>
struct BwdRows {
    static constexpr int RS = D + 8;     // padded row (bf16): rows 4 banks apart
    static constexpr int TS = kBM + 8;   // padded transposed row (bf16)
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// LDS row of item j (of a 64-item chunk) in the row-major buffers of the
// fused kernel. A score tile (block kb, half h) reads item
// 32 kb + 8 a + 4 h + b in lane 4 a + b; storing that item at row
// 32 kb + 16 h + 4 a + b makes the 16 lanes of a tile read 16 consecutive
// rows (rows 4 banks apart), where the item order would put rows 8 items
// apart on the same banks.
__device__ __forceinline__ int phys_row(int j) {
    return (j & ~31) | (((j >> 3) & 3) << 2) | (((j >> 2) & 1) << 4) | (j & 3);
}

// Transposes the 64 rows of `rm` (stored at phys_row(item)) into `tr`
// ([D][TS], item order) inside LDS. The 64 lanes of a wave take the 64 items
// at one 8-feature piece: the 16-byte reads land on distinct banks and each
// of the 8 two-byte writes covers 128 contiguous bytes of a transposed row.
template <int D, int NT>
__device__ __forceinline__ void transpose_items(const uint16_t (*rm)[BwdRows<D>::RS],
                                                uint16_t (*tr)[BwdRows<D>::TS]) {
    const int item = threadIdx.x & (kBM - 1);
    const int row = phys_row(item);
    for (int pc = threadIdx.x >> 6; pc < D / 8; pc += NT / kBM) {
        const u32x4 a = *(const u32x4*)&rm[row][pc * 8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            tr[pc * 8 + e][item] = (uint16_t)((a[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    }
}

// ---------------------------------------------------------------------------
// Run-based matrix-core pass. A workgroup walks a run of run_len consecutive
// chunks of one (batch, head, round) segment. Chunk c's slots are the queries
// of the pairs (c, c - 1), (c, c) and the keys of the pairs (c, c), (c + 1, c).
// Eight waves: waves 0-3 take the query side, waves 4-7 the key side, so each
// SIMD runs one of each and the matrix work of one overlaps the other's
// vector work. At step c
//   query waves: chunk c as queries against the keys of chunks c - 1 and c
//                (dq), handed to the key waves through LDS (bf16);
//   key waves:   chunk c - 1 as keys against chunk c's queries (the key side
//                of pair (c, c - 1)), then chunk c - 1's rows out
//                ((dq + dk) scaled, dv); chunk c as keys against its own
//                queries (dk, dv so far).
// LDS holds the rows of chunks c - 1 and c (qk and v row-major, qk
// transposed, one slot per chunk parity) and chunk c's output gradients.
// Chunk c + 1's rows are gathered into registers at the top of step c and
// parked in the slot chunk c - 1 leaves, so every chunk's rows come from HBM
// once per run and a gather has a whole step of matrix work to arrive. The
// last chunk of a run is finished by a partial step on the next chunk (its
// key side only), whose run repeats that pair for its own queries.
constexpr int kBwdThreads = 512;

// Chunks per workgroup: longer runs repeat the partial step on the next chunk
// and the first gather's wait less often (64 chunks: 3 % less backward time
// than 16 at 64K tokens x 8 heads x 8 rounds), as long as the grid keeps at
// least four workgroups per compute unit; never fewer than 16.
inline int bwd_run_len(int64_t segs, int nchunks) {
    constexpr int64_t kMinGrid = 4 * 256;
    int run = 64;
    while (run > 16 && segs * ((nchunks + run - 1) / run) < kMinGrid) run /= 2;
    return run;
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

template <int D>
struct alignas(16) BwdRunLds {
    static constexpr int RS = BwdRows<D>::RS, TS = BwdRows<D>::TS;
    uint16_t xr[2][kBM][RS];   // qk rows of the chunk of each parity (phys_row order)
    uint16_t vr[2][kBM][RS];   // v rows
    uint16_t gr[kBM][RS];      // output-gradient rows of the current chunk
    uint16_t xt[2][D][TS];     // qk transposed (item order)
    uint16_t gt[D][TS];        // output gradients transposed
    uint16_t xq[kBM][RS];      // dq of the current chunk (bf16), query waves -> key waves
    int32_t pos[3][kBM], bkt[3][kBM];          // chunk t in slot t % 3
    float zz[2][kBM], dd[2][kBM], rn[2][kBM];   // chunk t in slot t & 1
};

template <int D, bool PACKED, bool KN>
__global__ __launch_bounds__(kBwdThreads) void bwd_run_kernel(const uint16_t* __restrict__ qk,
                                                              const uint16_t* __restrict__ v,
                                                              const uint16_t* __restrict__ g,
                                                              const int32_t* __restrict__ perm,
                                                              const int32_t* __restrict__ buckets,
                                                              const float* __restrict__ z,
                                                              const float* __restrict__ Dv,
                                                              const float* __restrict__ rn, Dims dm,
                                                              int nruns, int run_len,
                                                              uint16_t* __restrict__ dx_r,
                                                              uint16_t* __restrict__ dv_r) {
    constexpr int KSTEPS = D / 32, DT = D / 16;
    constexpr int PER = kBM * (D / 8) / kBwdThreads;   // 16-byte pieces per thread and source
    static_assert(PER >= 1, "every thread moves a piece of each row set");
    __shared__ BwdRunLds<D> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool qside = wave < 4;   // waves 0-3: query side; 4-7: key side
    const int wg = wave & 3;       // the wave's 16 slots in a chunk
    const int gq = lane >> 4, r16 = lane & 15;
    const int64_t seg = blockIdx.x / nruns;
    const int run = blockIdx.x - (int)(seg * nruns);
    const int nchunks = dm.L / kBM;
    const int c0 = run * run_len;
    const int c1 = min(c0 + run_len, nchunks);
    const int clast = min(c1, nchunks - 1);   // step c1 (when it exists) is key side only
    const int64_t L = dm.L;
    const int64_t bh = seg / dm.nh;
    const int r = (int)(seg - bh * dm.nh);
    const int32_t* P = perm + seg * L;
    const int32_t* Bk = buckets + seg * L;
    const uint16_t* X = qk + bh * L * D;
    const uint16_t* V = v + bh * L * D;
    const uint16_t* G = g + bh * L * D;
    const float c2 = kLog2e / sqrtf((float)D);
    const float pen2 = kSelfPenalty * kLog2e;
    const float inv_nh = 1.0f / (float)dm.nh;
    const float scale = 1.0f / sqrtf((float)D);
    const int me = 16 * wg + r16;   // this lane's slot within a chunk
    const int prow = phys_row(me);

    // rows of chunk t (positions in its pos slot) into registers, then LDS
    struct Pre {
        u32x4 x[PER], v[PER], g[PER];
        float z, d, rn;
    };
    auto gather = [&](int t, Pre& pf) {
        const int s3 = t % 3;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + kBwdThreads * k, row = i / (D / 8), pc = i % (D / 8);
            const int64_t off = (int64_t)sm.pos[s3][row] * D + pc * 8;
            pf.x[k] = *(const u32x4*)(X + off);
            pf.v[k] = *(const u32x4*)(V + off);
            pf.g[k] = *(const u32x4*)(G + off);
        }
        if (tid < kBM) {
            const int64_t p = bh * L + sm.pos[s3][tid];
            pf.z = z[p];
            pf.d = Dv[p];
            pf.rn = KN ? rn[p] : 1.f;
        }
    };
    auto park = [&](int t, const Pre& pf) {
        const int par = t & 1;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + kBwdThreads * k, row = phys_row(i / (D / 8)), pc = i % (D / 8);
            *(u32x4*)&sm.xr[par][row][pc * 8] = pf.x[k];
            *(u32x4*)&sm.vr[par][row][pc * 8] = pf.v[k];
            *(u32x4*)&sm.gr[row][pc * 8] = pf.g[k];
        }
        if (tid < kBM) {
            sm.zz[par][tid] = pf.z;
            sm.dd[par][tid] = pf.d;
            sm.rn[par][tid] = pf.rn;
        }
    };
    auto load_keys = [&](int t) {   // sorted keys of chunk t into its slot (threads < 64)
        int32_t p, b;
        read_key<PACKED>(P, Bk, (int64_t)t * kBM + tid, p, b);
        sm.pos[t % 3][tid] = p;
        sm.bkt[t % 3][tid] = b;
    };

    // A 32-item block takes part only if its bucket range meets the wave's
    // (chunks are sorted by bucket) and, within one chunk under causality,
    // only if it is not wholly on the wrong side: a key slot after every
    // query slot of the same bucket has a later position. Wave-uniform.
    auto active = [&](int lo, int hi, int mlo, int mhi, bool skip) -> bool {
        const bool a = lo <= mhi && hi >= mlo && !skip;
        return __builtin_amdgcn_readfirstlane((int)a) != 0;
    };
    // chunk c's queries (fragments xf, gf) against the keys of chunk t (LDS)
    auto query_pass = [&](int t, bool own, const bf16x8(&xf)[KSTEPS], const bf16x8(&gf)[KSTEPS],
                          int32_t mpos, int32_t mbkt, float mz2, float mD, bool mself_only,
                          int mlo, int mhi, f32x4(&dq)[DT]) {
        const int par = t & 1, s3 = t % 3;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (!active(sm.bkt[s3][32 * kb], sm.bkt[s3][32 * kb + 31], mlo, mhi,
                        own && dm.causal && 32 * kb > 16 * wg + 15))
                continue;
            u32x4 dsfrag;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // tile row r16 is item 32 kb + 8 (r16 / 4) + 4 h + r16 % 4
                const int kw = 32 * kb + 16 * h + r16;   // its LDS row
                f32x4 sacc = {0.f, 0.f, 0.f, 0.f}, pacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KSTEPS; ++s) {
                    const bf16x8 ka = __builtin_bit_cast(bf16x8, *(const u32x4*)&sm.xr[par][kw][32 * s + 8 * gq]);
                    const bf16x8 va = __builtin_bit_cast(bf16x8, *(const u32x4*)&sm.vr[par][kw][32 * s + 8 * gq]);
                    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, xf[s], sacc, 0, 0, 0);
                    pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, gf[s], pacc, 0, 0, 0);
                }
                float ds[4];
                const int kbase = 32 * kb + 8 * gq + 4 * h;   // register i is key kbase + i
                const i32x4 kps = *(const i32x4*)&sm.pos[s3][kbase];
                const i32x4 kbk = *(const i32x4*)&sm.bkt[s3][kbase];
                f32x4 krn = {1.f, 1.f, 1.f, 1.f};
                if constexpr (KN) krn = *(const f32x4*)&sm.rn[par][kbase];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool ok = kbk[i] == mbkt && (!dm.causal || kps[i] <= mpos);
                    const float s2 = sacc[i] * krn[i] * c2 - (kps[i] == mpos ? pen2 : 0.f);
                    const float pw = pair_weight(ok, kps[i] == mpos, s2, mz2, mself_only, inv_nh);
                    ds[i] = pw * (pacc[i] - mD) * krn[i];
                }
                dsfrag[2 * h] = pack_bf16x2(ds[0], ds[1]);
                dsfrag[2 * h + 1] = pack_bf16x2(ds[2], ds[3]);
            }
            const bf16x8 bd = __builtin_bit_cast(bf16x8, dsfrag);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8 af = __builtin_bit_cast(
                    bf16x8, *(const u32x4*)&sm.xt[par][dt * 16 + r16][32 * kb + 8 * gq]);
                dq[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bd, dq[dt], 0, 0, 0);
            }
        }
    };
    // keys in fragments (xf, vf) against the queries of chunk t (LDS, with
    // its output gradients in gr / gt)
    auto key_pass = [&](int t, bool own, const bf16x8(&xf)[KSTEPS], const bf16x8(&vf)[KSTEPS],
                        int32_t mpos, int32_t mbkt, float mrn, int mlo, int mhi,
                        f32x4(&dk)[DT], f32x4(&dvv)[DT], float& msdd) {
        const int par = t & 1, s3 = t % 3;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            if (!active(sm.bkt[s3][32 * qb], sm.bkt[s3][32 * qb + 31], mlo, mhi,
                        own && dm.causal && 32 * qb + 31 < 16 * wg))
                continue;
            u32x4 pfrag, dsfrag;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int qw = 32 * qb + 16 * h + r16;
                f32x4 sacc = {0.f, 0.f, 0.f, 0.f}, pacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KSTEPS; ++s) {
                    const bf16x8 qa = __builtin_bit_cast(bf16x8, *(const u32x4*)&sm.xr[par][qw][32 * s + 8 * gq]);
                    const bf16x8 ga = __builtin_bit_cast(bf16x8, *(const u32x4*)&sm.gr[qw][32 * s + 8 * gq]);
                    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, xf[s], sacc, 0, 0, 0);
                    pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga, vf[s], pacc, 0, 0, 0);
                }
                float pw[4], ds[4];
                const int qbase = 32 * qb + 8 * gq + 4 * h;   // register i is query qbase + i
                const i32x4 qps = *(const i32x4*)&sm.pos[s3][qbase];
                const i32x4 qbk = *(const i32x4*)&sm.bkt[s3][qbase];
                const f32x4 zq = *(const f32x4*)&sm.zz[par][qbase];
                const f32x4 dq4 = *(const f32x4*)&sm.dd[par][qbase];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool ok = qbk[i] == mbkt && (!dm.causal || mpos <= qps[i]);
                    const float s2 = sacc[i] * mrn * c2 - (mpos == qps[i] ? pen2 : 0.f);
                    pw[i] = pair_weight(ok, mpos == qps[i], s2, zq[i] * kLog2e,
                                        zq[i] < -0.5f * kSelfPenalty, inv_nh);
                    ds[i] = pw[i] * (pacc[i] - dq4[i]);
                    if constexpr (KN) msdd = fmaf(ds[i], sacc[i], msdd);
                }
                pfrag[2 * h] = pack_bf16x2(pw[0], pw[1]);
                pfrag[2 * h + 1] = pack_bf16x2(pw[2], pw[3]);
                dsfrag[2 * h] = pack_bf16x2(ds[0], ds[1]);
                dsfrag[2 * h + 1] = pack_bf16x2(ds[2], ds[3]);
            }
            const bf16x8 bp = __builtin_bit_cast(bf16x8, pfrag);
            const bf16x8 bd = __builtin_bit_cast(bf16x8, dsfrag);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8 aq = __builtin_bit_cast(
                    bf16x8, *(const u32x4*)&sm.xt[par][dt * 16 + r16][32 * qb + 8 * gq]);
                const bf16x8 ag = __builtin_bit_cast(
                    bf16x8, *(const u32x4*)&sm.gt[dt * 16 + r16][32 * qb + 8 * gq]);
                dk[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bd, dk[dt], 0, 0, 0);
                dvv[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag, bp, dvv[dt], 0, 0, 0);
            }
        }
    };
    // rows (dq + dk) * scale and dv of one slot; lane (slot, gq) holds
    // features 16 dt + 4 gq + i of dk and dv, and dq waits in xq (the query
    // waves write the next chunk's only after the barrier that ends this pass)
    auto write_out = [&](int32_t mpos, float mrn, float msdd, f32x4(&dk)[DT], f32x4(&dvv)[DT]) {
        const int64_t row = ((bh * L + mpos) * dm.nh + r) * D;
        if constexpr (KN) {
            // dk = rn (sum dS x_i - rn^2 (sum dS x_i . x_j) x_j); the lanes of a
            // slot hold disjoint query sets, so their sums are added first
            msdd += __shfl_xor(msdd, 16);
            msdd += __shfl_xor(msdd, 32);
            const float pr = mrn * mrn * msdd;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const uint2 w = *(const uint2*)(X + (int64_t)mpos * D + 16 * dt + 4 * gq);
                const f32x4 xm = {__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                                  __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
                dk[dt] = (dk[dt] - pr * xm) * mrn;
            }
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const uint2 w = *(const uint2*)&sm.xq[me][16 * dt + 4 * gq];
            const f32x4 dq = {__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                              __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
            const f32x4 a = (dq + dk[dt]) * scale;
            const f32x4 b = dvv[dt];
            *(uint2*)(dx_r + row + 16 * dt + 4 * gq) =
                make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
            *(uint2*)(dv_r + row + 16 * dt + 4 * gq) =
                make_uint2(pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3]));
        }
    };

    // ---- prologue: sorted keys of chunks c0 - 1 .. c0 + 1, rows of chunks
    // c0 - 1 and c0 (and their transposes)
    if (tid < kBM)
        for (int t = max(c0 - 1, 0); t <= min(c0 + 1, clast); ++t) load_keys(t);
    __syncthreads();
    Pre pf;
    if (c0 > 0) {
        gather(c0 - 1, pf);
        park(c0 - 1, pf);
    }
    gather(c0, pf);
    park(c0, pf);   // the same thread overwrites the output-gradient rows
    __syncthreads();
    if (c0 > 0) transpose_items<D, kBwdThreads>(sm.xr[(c0 - 1) & 1], sm.xt[(c0 - 1) & 1]);
    transpose_items<D, kBwdThreads>(sm.xr[c0 & 1], sm.xt[c0 & 1]);
    transpose_items<D, kBwdThreads>(sm.gr, sm.gt);
    __syncthreads();

    // One set of variables, two roles: query waves keep chunk c's qk and
    // output-gradient fragments (fa, fb) and dq (acc); key waves keep their
    // key chunk's qk and v fragments (fa, fb), dk (acc) and dv (acc2),
    // carried into the next step, where the key side of pair (c + 1, c)
    // finishes them.
    bf16x8 fa[KSTEPS], fb[KSTEPS];
    f32x4 acc[DT], acc2[DT];
    int32_t mpos = 0, mbkt = -1;
    float mrn = 1.f, msdd = 0.f;
    for (int c = c0; c <= clast; ++c) {
        const bool mine = c < c1;          // chunk c belongs to this run
        const bool nxt = c + 1 <= clast;   // chunk c + 1 is stepped by this run
        const int par = c & 1, s3 = c % 3;
        // sorted keys of chunk c + 2 and rows of chunk c + 1 start travelling
        int32_t kp2 = 0, kb2 = -1;
        if (tid < kBM && c + 2 <= clast) read_key<PACKED>(P, Bk, (int64_t)(c + 2) * kBM + tid, kp2, kb2);
        if (nxt) gather(c + 1, pf);
        const int mlo = sm.bkt[s3][16 * wg], mhi = sm.bkt[s3][16 * wg + 15];
        if (qside) {
            if (mine) {
                // chunk c as queries against chunks c - 1 and c
#pragma unroll
                for (int s = 0; s < KSTEPS; ++s) {
                    fa[s] = __builtin_bit_cast(bf16x8, *(const u32x4*)&sm.xr[par][prow][32 * s + 8 * gq]);
                    fb[s] = __builtin_bit_cast(bf16x8, *(const u32x4*)&sm.gr[prow][32 * s + 8 * gq]);
                }
                mpos = sm.pos[s3][me];
                mbkt = sm.bkt[s3][me];
                const float mz = sm.zz[par][me], mD = sm.dd[par][me];
                const bool self_only = mz < -0.5f * kSelfPenalty;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
                if (c > 0)
                    query_pass(c - 1, false, fa, fb, mpos, mbkt, mz * kLog2e, mD, self_only, mlo, mhi, acc);
                query_pass(c, true, fa, fb, mpos, mbkt, mz * kLog2e, mD, self_only, mlo, mhi, acc);
            }
        } else {
            // chunk c - 1 as keys against chunk c's queries, then its rows out
            if (c > c0) {
                const int s3p = (c - 1) % 3;   // chunk c - 1's keys: this wave's bucket range
                key_pass(c, false, fa, fb, mpos, mbkt, mrn, sm.bkt[s3p][16 * wg],
                         sm.bkt[s3p][16 * wg + 15], acc, acc2, msdd);
                write_out(mpos, mrn, msdd, acc, acc2);
            }
            if (mine) {
                // chunk c as keys against its own queries
#pragma unroll
                for (int s = 0; s < KSTEPS; ++s) {
                    fa[s] = __builtin_bit_cast(bf16x8, *(const u32x4*)&sm.xr[par][prow][32 * s + 8 * gq]);
                    fb[s] = __builtin_bit_cast(bf16x8, *(const u32x4*)&sm.vr[par][prow][32 * s + 8 * gq]);
                }
                mpos = sm.pos[s3][me];
                mbkt = sm.bkt[s3][me];
                mrn = KN ? sm.rn[par][me] : 1.f;
                msdd = 0.f;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[dt] = acc2[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
                key_pass(c, true, fa, fb, mpos, mbkt, mrn, mlo, mhi, acc, acc2, msdd);
            }
        }
        __syncthreads();   // chunk c - 1's slot, chunk c's gradients and xq (read by the write-out) are free
        if (qside && mine) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *(uint2*)&sm.xq[me][16 * dt + 4 * gq] =
                    make_uint2(pack_bf16x2(acc[dt][0], acc[dt][1]), pack_bf16x2(acc[dt][2], acc[dt][3]));
        }
        if (nxt) {
            park(c + 1, pf);
            if (tid < kBM && c + 2 <= clast) {
                sm.pos[(c + 2) % 3][tid] = kp2;
                sm.bkt[(c + 2) % 3][tid] = kb2;
            }
        }
        __syncthreads();
        if (nxt) {
            transpose_items<D, kBwdThreads>(sm.xr[(c + 1) & 1], sm.xt[(c + 1) & 1]);
            transpose_items<D, kBwdThreads>(sm.gr, sm.gt);
        }
        __syncthreads();
    }
    // a run that ends its segment finishes its last chunk here: there is no
    // pair (c1, c1 - 1)
    if (!qside && c1 == nchunks) write_out(mpos, mrn, msdd, acc, acc2);
}

template <int D, typename T, bool PACKED>
hipError_t launch_bwd_t(const BwdArgs& a, const Dims& d, hipStream_t st) {
    const T* qk = (const T*)a.qk;
    const T* v = (const T*)a.v;
    const T* g = (const T*)a.dout;
    if constexpr (sizeof(T) == 2) {
        const unsigned gq = (unsigned)((d.T * (D / 8) + 255) / 256);
        bwd_dot_bf16_kernel<D><<<gq, 256, 0, st>>>(g, (const T*)a.out, d, a.Dv);
    } else {
        const unsigned gq = (unsigned)((d.T * 4 + 255) / 256);
        bwd_dot_kernel<D, T><<<gq, 256, 0, st>>>(g, (const T*)a.out, d, a.Dv);
    }
    if constexpr (sizeof(T) == 2) {
        if (d.m == kBM) {   // matrix-core passes
            uint16_t* hx = (uint16_t*)a.dx_r;
            uint16_t* hv = (uint16_t*)a.dv_r;
            const int nchunks = d.L / kBM;
            const int run_len = bwd_run_len(d.segs, nchunks);
            const int nruns = (nchunks + run_len - 1) / run_len;
            const unsigned grid = (unsigned)(d.segs * nruns);
            if (a.rn)
                bwd_run_kernel<D, PACKED, true><<<grid, kBwdThreads, 0, st>>>(
                    qk, v, g, a.perm, a.buckets, a.z, a.Dv, a.rn, d, nruns, run_len, hx, hv);
            else
                bwd_run_kernel<D, PACKED, false><<<grid, kBwdThreads, 0, st>>>(
                    qk, v, g, a.perm, a.buckets, a.z, a.Dv, nullptr, d, nruns, run_len, hx, hv);
            const unsigned gr = (unsigned)((d.T * (D / 8) + 255) / 256);
            bwd_reduce_bf16_kernel<D><<<gr, 256, 0, st>>>(hx, hv, d, (uint16_t*)a.dqk,
                                                          (uint16_t*)a.dv);
            return hipGetLastError();
        }
    }
    const int nqb = (d.m + 63) / 64;
    const dim3 grid((unsigned)((int64_t)(d.L / d.m) * nqb), (unsigned)d.segs);
    bwd_dq_kernel<D, T, PACKED><<<grid, 256, 0, st>>>(qk, v, g, a.perm, a.buckets, a.z, a.Dv,
                                                      a.rn, d, nqb, a.dx_r);
    bwd_dkv_kernel<D, T, PACKED><<<grid, 256, 0, st>>>(qk, v, g, a.perm, a.buckets, a.z, a.Dv,
                                                       a.rn, d, nqb, a.dx_r, a.dv_r);
    const unsigned gr = (unsigned)((d.T * (D / 4) + 255) / 256);
    bwd_reduce_kernel<D, T, float><<<gr, 256, 0, st>>>(a.dx_r, a.dv_r, d, (T*)a.dqk, (T*)a.dv);
    return hipGetLastError();
}

template <typename T, bool PACKED>
hipError_t launch_bwd_d(const BwdArgs& a, const Dims& d, hipStream_t st) {
    return d.d == 64 ? launch_bwd_t<64, T, PACKED>(a, d, st) : launch_bwd_t<128, T, PACKED>(a, d, st);
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, const Dims& d, bool packed, hipStream_t st) {
    if (d.T == 0) return hipSuccess;
    if (d.key_norm != (a.rn != nullptr)) return hipErrorInvalidValue;
    if (d.dtype == LSH_BF16)
        return packed ? launch_bwd_d<uint16_t, true>(a, d, st) : launch_bwd_d<uint16_t, false>(a, d, st);
    return packed ? launch_bwd_d<float, true>(a, d, st) : launch_bwd_d<float, false>(a, d, st);
}

}  // namespace lsh
