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
// Every operand is formed and the result selected, without branches: the
// pairs of a wave take different cases, and a branch per pair would
// serialise them.
__device__ __forceinline__ float pair_weight(bool ok, bool self, float s2, float z2,
                                             bool self_only, float inv_nh) {
    const float e = __builtin_amdgcn_exp2f(s2 - z2);
    const float w = self_only ? (self ? inv_nh : 0.f) : e;
    return ok ? w : 0.f;
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
    const int64_t seg = block_y();
    if (seg >= dm.segs) return;
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
    const int64_t seg = block_y();
    if (seg >= dm.segs) return;
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
// read once), fp32 sums. Blocks run from the last token back: the matrix-core
// pass writes the last (batch, head) slices' rows last, and those are still
// in the memory-side cache when this pass starts.
template <int D>
__global__ __launch_bounds__(256) void bwd_reduce_bf16_kernel(const uint16_t* __restrict__ dx_r,
                                                              const uint16_t* __restrict__ dv_r,
                                                              Dims dm, uint16_t* __restrict__ dqk,
                                                              uint16_t* __restrict__ dv) {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    const int64_t gid = (int64_t)(gridDim.x - 1 - blockIdx.x) * blockDim.x + threadIdx.x;
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
    // qk and output-gradient rows (bf16): rows 8 banks apart, and rows whose
    // index has bit 3 set 4 banks further on. 16 consecutive rows read 16
    // bytes each at one column (a score tile's A operand) then cover the 64
    // banks once, and so do 8 consecutive rows read 8 bytes each at four
    // neighbouring 4-column chunks (a transposing read of 32 lanes).
    static constexpr int XS = D + 16;
    static constexpr int xrow(int r) { return r * XS + 8 * ((r >> 3) & 1); }
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// LDS row of item j (of a 64-item chunk) in the row-major buffers of the
// fused kernel. A score tile (block kb, half h) reads item
// 32 kb + 8 a + 4 h + b in lane 4 a + b; storing that item at row
// 32 kb + 16 h + 4 a + b makes the 16 lanes of a tile read 16 consecutive
// rows (rows 4 banks apart), where the item order would put rows 8 items
// apart on the same banks.
__device__ __forceinline__ int phys_row(int j) {
    return (j & ~31) | (((j >> 3) & 3) << 2) | (((j >> 2) & 1) << 4) | (j & 3);
}

// A transposed operand straight from row-major rows: the A operand of a
// 16 x 16 x 32 product whose rows m are 16 features and whose k runs over
// the items 32 kb + 8 gq + e (e < 8) of a row buffer laid out by phys_row
// and xrow. Items 8 gq + 0 .. 3 of a block sit on four consecutive rows
// (4 gq .. 4 gq + 3), items 8 gq + 4 .. 7 on the four rows 16 further on.
// ds_read_b64_tr_b16 hands lane j of a 16-lane group element j % 4 of the
// 8-byte pieces that lanes j / 4 + 4 i (i < 4) address: with lane r16 of
// group gq addressing row 4 gq + r16 / 4 at columns 4 (r16 % 4) .. + 3, lane
// r16 receives column r16 of those four rows, k-elements 0 .. 3, and the
// read 16 rows on gives elements 4 .. 7. `p` is that lane's address in the
// block (tile column 0).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* p) {
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 16 * BwdRows<D>::XS));
    const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(bf16x8, (u32x4){a.x, a.y, b.x, b.y});
}

// ---------------------------------------------------------------------------
// Run-based matrix-core pass. A workgroup walks a run of run_len consecutive
// chunks of one (batch, head, round) segment. The keys of chunk t meet the
// queries of chunks t (own pair) and t + 1 (look-back pair), so eight waves
// split into two sets of four that take turns: at step c one set owns the 64
// keys of chunk c, the other those of chunk c - 1, each wave 16 of them, with
// their qk and v fragments and their dk, dv accumulators in registers for
// both of the chunk's steps. At step c every wave
//   A: scores its 16 keys against chunk c's 64 queries (S and dP tiles with
//      the queries' rows from LDS), forms the pair weights P and dS in the
//      lanes of its keys, adds dk += dS^T x_q and dv += P^T g_q (the queries'
//      rows from LDS, read transposed), and writes its dS (times the key's
//      1/|x| under key normalisation) into a [query][key] LDS buffer;
//   B: the set owning chunk c - 1 writes that chunk's rows out ((dq + dk)
//      scaled, and dv; its dq has waited in LDS since step c - 1), while the
//      set owning chunk c computes chunk c's dq = dS x_k over the 128 keys
//      (the keys' rows, read transposed, and the dS buffer from LDS) into
//      the other dq slot;
//   C: chunk c + 1's rows, gathered into registers since the top of the
//      step, are parked in LDS;
//   D: the set that just wrote chunk c - 1 out takes chunk c + 1's keys and
//      goes straight on to step c + 1 (it reads nothing the next step's A
//      writes, and the next writes to what it reads follow that step's
//      first barrier).
// Three barriers a step. The qk rows of chunks c - 1 and c stay in a
// two-slot ring, so the operands that run over queries or keys (x^T, g^T)
// come from the row-major rows by transposing reads, with no transposed
// copy and no pass to make one.
// Every score is computed once. The first step of a run scores the look-back
// pair for dq only (the run before finishes that chunk's dk, dv); a run that
// does not end its segment closes with a partial step on the next chunk
// (look-back keys only, no dq), whose run repeats those scores for its dq.
constexpr int kBwdThreads = 512;

// Chunks per workgroup: longer runs repeat the partial step on the next chunk
// and the first gather's wait less often, as long as the grid keeps at least
// four workgroups per compute unit; never fewer than 16.
inline int bwd_run_len(int64_t segs, int nchunks) {
    constexpr int64_t kMinGrid = 4 * 256;
    int run = 64;
    while (run > 16 && segs * ((nchunks + run - 1) / run) < kMinGrid) run /= 2;
    return run;
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// The dS buffer holds, for each of the 64 queries of a step, the 128 keys
// (chunk c - 1 then chunk c) as 16 units of 8 keys (16 bytes). Rows are 272
// bytes apart, with 32 more bytes after every 16 rows, so unit u of query q
// starts on bank 4 ((u + q + 2 (q / 16)) mod 16) of 64: the 16 lanes of a
// 16-byte read (16 consecutive queries at one unit) cover every bank once,
// and a dS write's 64 lanes (4 queries 8 apart, two units each) take 32
// distinct banks.
constexpr int kDsRow = 136;   // bf16 elements per row: 16 units and one unit of padding
constexpr int kDsGap = 16;    // bf16 elements after every 16 rows

template <int D>
struct alignas(16) BwdRunLds {
    static constexpr int RS = BwdRows<D>::RS;
    static constexpr int XS = BwdRows<D>::XS;
    // qk rows of chunk t in slot t & 1 (item j at row phys_row(j), row r at xrow(r))
    uint16_t xr[2][kBM * XS];
    uint16_t gr[kBM * XS];     // output-gradient rows of chunk c (same layout)
    uint16_t vr[kBM][RS];      // v rows of chunk c (phys_row order)
    uint16_t ds[kBM * kDsRow + (kBM / 16) * kDsGap];   // dS of step c by [query][key]
    uint16_t xq[2][kBM][RS];   // dq of chunk t in slot t & 1 (bf16, item order)
    int32_t pos[3][kBM], bkt[3][kBM];   // chunk t in slot t % 3
    float zz[kBM], dd[kBM], rn[kBM];    // chunk c's Z, D and 1 / |x|
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
    constexpr int DPW = DT / 4;   // dq feature tiles (of 16) per wave of the set computing dq
    static_assert(PER >= 1, "every thread moves a piece of each row set");
    __shared__ BwdRunLds<D> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wset = wave >> 2;    // the set: owns chunks t with t & 1 == wset
    const int wg = wave & 3;       // the wave's 16 keys in a chunk
    const int gq = lane >> 4, r16 = lane & 15;
    const int64_t seg = blockIdx.x / nruns;
    const int run = blockIdx.x - (int)(seg * nruns);
    const int nchunks = dm.L / kBM;
    const int c0 = run * run_len;
    const int c1 = min(c0 + run_len, nchunks);
    const int clast = min(c1, nchunks - 1);   // step c1 (when it exists) is a partial step
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
    const int me = 16 * wg + r16;   // this lane's key within its chunk
    const int prow = phys_row(me);
    // Per-lane LDS addresses; every tile below is a constant offset from one
    // of them: row r16 at column 8 gq for the row reads, row 4 gq + r16 / 4
    // at column 4 (r16 % 4) for the transposing reads (tr_operand).
    constexpr int XS = BwdRows<D>::XS, SLOT = kBM * XS;
    const uint16_t* const xr_l = sm.xr[0] + BwdRows<D>::xrow(r16) + 8 * gq;
    const uint16_t* const gr_l = sm.gr + BwdRows<D>::xrow(r16) + 8 * gq;
    const int trow = 4 * gq + (r16 >> 2);
    const uint16_t* const xtr_l = sm.xr[0] + BwdRows<D>::xrow(trow) + 4 * (r16 & 3);
    const uint16_t* const gtr_l = sm.gr + BwdRows<D>::xrow(trow) + 4 * (r16 & 3);
    const uint16_t* const xtq_l = xtr_l + 16 * DPW * wg;   // this wave's first dq feature tile
    // dS writes: query 32 qb + 8 gq + e, key me (+ 64 for chunk c's keys)
    uint16_t* const dsw_l = &sm.ds[8 * gq * kDsRow + (gq >> 1) * kDsGap + me];
    // dS reads: query 16 qt + r16, keys 32 kb + 8 gq .. + 7
    const uint16_t* const dsr_l = &sm.ds[r16 * kDsRow + 8 * gq];

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
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + kBwdThreads * k, row = phys_row(i / (D / 8)), pc = i % (D / 8);
            *(u32x4*)(sm.xr[t & 1] + BwdRows<D>::xrow(row) + pc * 8) = pf.x[k];
            *(u32x4*)&sm.vr[row][pc * 8] = pf.v[k];
            *(u32x4*)(sm.gr + BwdRows<D>::xrow(row) + pc * 8) = pf.g[k];
        }
        if (tid < kBM) {
            sm.zz[tid] = pf.z;
            sm.dd[tid] = pf.d;
            sm.rn[tid] = pf.rn;
        }
    };
    auto load_keys = [&](int t) {   // sorted keys of chunk t into its slot (threads < 64)
        int32_t p, b;
        read_key<PACKED>(P, Bk, (int64_t)t * kBM + tid, p, b);
        sm.pos[t % 3][tid] = p;
        sm.bkt[t % 3][tid] = b;
    };

    // the wave's keys: fragments, position, bucket, 1 / |x|, accumulators
    bf16x8 kf[KSTEPS], vf[KSTEPS];
    f32x4 dk[DT], dvv[DT];
    int32_t mpos = 0, mbkt = -1;
    float mrn = 1.f, msdd = 0.f;
    // take the keys of chunk t (its rows parked in xr, vr; its keys in slot t % 3)
    auto take_keys = [&](int t) {
        const uint16_t* const xk = sm.xr[t & 1] + BwdRows<D>::xrow(prow) + 8 * gq;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            kf[s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(xk + 32 * s));
            vf[s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(&sm.vr[prow][8 * gq] + 32 * s));
        }
        mpos = sm.pos[t % 3][me];
        mbkt = sm.bkt[t % 3][me];
        mrn = KN ? sm.rn[me] : 1.f;
        msdd = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) dk[dt] = dvv[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    };

    // Phase A for this wave's keys (of chunk c when own, else c - 1) against
    // chunk c's queries. Tile rows are queries: A-row m of block qb, half h
    // is query 32 qb + 8 (m / 4) + 4 h + m % 4 (LDS row 32 qb + 16 h + m), so
    // after both halves lane (r16, gq) holds its key's P and dS for queries
    // 32 qb + 8 gq + e, e < 8: the B operand of the dk and dv products.
    auto key_step = [&](int c, bool own, bool do_dkv, bool do_ds) {
        const int s3 = c % 3, par = c & 1;
        const int klo = __builtin_amdgcn_readlane(mbkt, 0);
        const int khi = __builtin_amdgcn_readlane(mbkt, 15);
        const uint16_t* const xrc = xr_l + par * SLOT;    // chunk c's qk rows
        const uint16_t* const xtc = xtr_l + par * SLOT;   // the same, transposing reads
        uint16_t* const dsw = dsw_l + (own ? kBM : 0);      // chunk c's keys: columns 64..127
        // both query blocks' bucket bounds first, then one wave-uniform mask
        // (non-short-circuit & and |: the loads are all issued before any test)
        int lo[2], hi[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            lo[qb] = sm.bkt[s3][32 * qb];
            hi[qb] = sm.bkt[s3][32 * qb + 31];
        }
        uint32_t act = 0;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const bool a = (lo[qb] <= khi) & (hi[qb] >= klo) &
                           !(own && dm.causal && 16 * wg > 32 * qb + 31);
            act |= (uint32_t)a << qb;
        }
        act = __builtin_amdgcn_readfirstlane(act);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            u32x4 pfrag = {0u, 0u, 0u, 0u}, dsfrag = {0u, 0u, 0u, 0u}, dqfrag = {0u, 0u, 0u, 0u};
            if ((act >> qb) & 1) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    f32x4 sacc = {0.f, 0.f, 0.f, 0.f}, pacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KSTEPS; ++s) {
                        // A row r16 of the tile: LDS row 32 qb + 16 h + r16
                        const int off = (32 * qb + 16 * h) * XS + 32 * s;
                        const bf16x8 qa = __builtin_bit_cast(bf16x8, *(const u32x4*)(xrc + off));
                        const bf16x8 ga = __builtin_bit_cast(bf16x8, *(const u32x4*)(gr_l + off));
                        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kf[s], sacc, 0, 0, 0);
                        pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga, vf[s], pacc, 0, 0, 0);
                    }
                    float pw[4], ds[4];
                    const int qbase = 32 * qb + 8 * gq + 4 * h;   // register i is query qbase + i
                    const i32x4 qps = *(const i32x4*)&sm.pos[s3][qbase];
                    const i32x4 qbk = *(const i32x4*)&sm.bkt[s3][qbase];
                    const f32x4 zq = *(const f32x4*)&sm.zz[qbase];
                    const f32x4 dq4 = *(const f32x4*)&sm.dd[qbase];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool ok = (qbk[i] == mbkt) & (!dm.causal | (mpos <= qps[i]));
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
                    if constexpr (KN) {   // dq takes dS times the key's 1 / |x|
                        dqfrag[2 * h] = pack_bf16x2(ds[0] * mrn, ds[1] * mrn);
                        dqfrag[2 * h + 1] = pack_bf16x2(ds[2] * mrn, ds[3] * mrn);
                    }
                }
                if (do_dkv) {
                    const bf16x8 bp = __builtin_bit_cast(bf16x8, pfrag);
                    const bf16x8 bd = __builtin_bit_cast(bf16x8, dsfrag);
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) {
                        const int off = 32 * qb * XS + 16 * dt;
                        const bf16x8 aq = tr_operand<D>(xtc + off);
                        const bf16x8 ag = tr_operand<D>(gtr_l + off);
                        dk[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bd, dk[dt], 0, 0, 0);
                        dvv[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag, bp, dvv[dt], 0, 0, 0);
                    }
                }
            }
            if (do_ds) {   // zeros for a skipped block: the dq pass reads every key block it keeps
                if constexpr (!KN) dqfrag = dsfrag;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    dsw[qb * (32 * kDsRow + 2 * kDsGap) + e * kDsRow] =
                        (uint16_t)(dqfrag[e >> 1] >> (16 * (e & 1)));
            }
        }
    };

    // Phase B, the set that owns chunk c's keys: dq^T tiles (16 features x
    // 16 queries) of chunk c over the keys of chunks c - 1 (blocks 0, 1) and c
    // (blocks 2, 3); wave wg takes feature tiles DPW wg .. + DPW - 1 of all
    // four query tiles. A: the keys' rows read transposed; B: lane (r16, gq) reads
    // keys 32 kb + 8 gq .. + 7 of query 16 qt + r16 from the dS buffer, each
    // read serving DPW products. Lane (r16, gq) of tile (u, qt) ends with
    // features 16 (DPW wg + u) + 4 gq + i of query 16 qt + r16, stored to xq.
    // Every tile is computed (a skipped block left zeros in the dS buffer):
    // without per-tile tests all operand reads issue ahead of the products.
    auto dq_pass = [&](int c) {
        f32x4 dqa[DPW][4];
#pragma unroll
        for (int u = 0; u < DPW; ++u)
#pragma unroll
            for (int qt = 0; qt < 4; ++qt) dqa[u][qt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (kb < 2 && c == 0) continue;   // no chunk before the first
            const int tk = kb < 2 ? c - 1 : c;
            bf16x8 ak[DPW];
#pragma unroll
            for (int u = 0; u < DPW; ++u)
                ak[u] = tr_operand<D>(xtq_l + (tk & 1) * SLOT + 32 * (kb & 1) * XS + 16 * u);
#pragma unroll
            for (int qt = 0; qt < 4; ++qt) {
                const bf16x8 bd = __builtin_bit_cast(
                    bf16x8, *(const u32x4*)(dsr_l + qt * (16 * kDsRow + kDsGap) + 32 * kb));
#pragma unroll
                for (int u = 0; u < DPW; ++u)
                    dqa[u][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[u], bd, dqa[u][qt], 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < DPW; ++u)
#pragma unroll
            for (int qt = 0; qt < 4; ++qt)
                *(uint2*)&sm.xq[c & 1][16 * qt + r16][16 * (DPW * wg + u) + 4 * gq] =
                    make_uint2(pack_bf16x2(dqa[u][qt][0], dqa[u][qt][1]),
                               pack_bf16x2(dqa[u][qt][2], dqa[u][qt][3]));
    };

    // Rows (dq + dk) * scale and dv of this wave's 16 keys (chunk t). Lane
    // (key, gq) holds features 16 dt + 4 gq + i of dk and dv, and dq waits in
    // xq. The finished rows are staged in LDS (dx over dq in xq, dv in vr,
    // which is parked again only after the next barrier) and stored 16 bytes
    // per lane with D / 8 lanes per row, so each store writes whole rows
    // instead of 32-byte pieces of 16 rows.
    auto write_out = [&](int t) {
        if constexpr (KN) {
            // dk = rn (sum dS x_i - rn^2 (sum dS x_i . x_j) x_j); the lanes of a
            // key hold disjoint query sets, so their sums are added first
            float sd = msdd;
            sd += __shfl_xor(sd, 16);
            sd += __shfl_xor(sd, 32);
            const float pr = mrn * mrn * sd;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const uint2 w = *(const uint2*)(X + (int64_t)mpos * D + 16 * dt + 4 * gq);
                const f32x4 xm = {__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                                  __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
                dk[dt] = (dk[dt] - pr * xm) * mrn;
            }
        }
        uint16_t* const xs = &sm.xq[t & 1][me][4 * gq];
        uint16_t* const vs = &sm.vr[me][4 * gq];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const uint2 w = *(const uint2*)(xs + 16 * dt);
            const f32x4 dq = {__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                              __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
            const f32x4 a = (dq + dk[dt]) * scale;
            const f32x4 b = dvv[dt];
            *(uint2*)(xs + 16 * dt) = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
            *(uint2*)(vs + 16 * dt) = make_uint2(pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3]));
        }
        // the wave's own rows only: its LDS writes above land before these reads
        constexpr int PCS = D / 8, RPI = 64 / PCS;   // 16-byte pieces per row, rows per store
        const int pc = lane % PCS;
#pragma unroll
        for (int k = 0; k < 16 / RPI; ++k) {
            const int item = 16 * wg + RPI * k + lane / PCS;
            const int64_t row = ((bh * L + sm.pos[t % 3][item]) * dm.nh + r) * D + 8 * pc;
            *(u32x4*)(dx_r + row) = *(const u32x4*)&sm.xq[t & 1][item][8 * pc];
            *(u32x4*)(dv_r + row) = *(const u32x4*)&sm.vr[item][8 * pc];
        }
    };

    // ---- prologue: sorted keys of chunks c0 - 1 .. c0 + 1; chunk c0 - 1's
    // keys to the set that owns it (for chunk c0's dq), then chunk c0's rows
    if (tid < kBM)
        for (int t = max(c0 - 1, 0); t <= min(c0 + 1, clast); ++t) load_keys(t);
    __syncthreads();
    Pre pf;
    if (c0 > 0) {
        gather(c0 - 1, pf);
        park(c0 - 1, pf);
        __syncthreads();
        if (wset == ((c0 - 1) & 1)) take_keys(c0 - 1);
        __syncthreads();   // v rows and 1 / |x| read before chunk c0's are parked
    }
    gather(c0, pf);
    park(c0, pf);
    __syncthreads();
    if (wset == (c0 & 1)) take_keys(c0);

    for (int c = c0; c <= clast; ++c) {
        const bool mine = c < c1;          // chunk c's queries belong to this run
        const bool nxt = c + 1 <= clast;   // chunk c + 1 is stepped by this run
        const bool own = wset == (c & 1);  // this wave's keys are chunk c's (else c - 1's)
        // sorted keys of chunk c + 2 and rows of chunk c + 1 start travelling
        int32_t kp2 = 0, kb2 = -1;
        if (tid < kBM && c + 2 <= clast) read_key<PACKED>(P, Bk, (int64_t)(c + 2) * kBM + tid, kp2, kb2);
        if (nxt) gather(c + 1, pf);
        // A
        if (own) {
            if (mine) key_step(c, true, true, true);
        } else if (c > 0) {
            key_step(c, false, c > c0, mine);
        }
        __syncthreads();   // the dS buffer is complete
        // B: one set writes chunk c - 1 out, the other computes chunk c's dq
        if (!own) {
            if (c > c0) write_out(c - 1);   // chunk c - 1 is finished
        } else if (mine) {
            dq_pass(c);
        }
        __syncthreads();   // the row buffers, chunk c - 1's keys slot and qk slot are free
        // C
        if (nxt) {
            park(c + 1, pf);
            if (tid < kBM && c + 2 <= clast) {
                sm.pos[(c + 2) % 3][tid] = kp2;
                sm.bkt[(c + 2) % 3][tid] = kb2;
            }
        }
        __syncthreads();
        // D
        if (nxt && !own) take_keys(c + 1);
    }
    // a run that ends its segment finishes its last chunk here: there is no
    // look-back pair for it
    if (c1 == nchunks && wset == ((c1 - 1) & 1)) write_out(c1 - 1);
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
    const dim3 grid = grid_split((unsigned)((int64_t)(d.L / d.m) * nqb), d.segs);
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
