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

// Plain fp32 kernel, for fp32 inputs and for any chunk length. A workgroup
// takes 64 query slots of one chunk; the four lanes of a query each hold a
// quarter of its features (dot products are summed across the quad). The
// window's keys pass through LDS 32 at a time and a running (online) softmax
// in the exp2 domain folds each block into the output.
//
// With separate queries and keys (SEP) the query of slot s comes from q
// through the queries' order (perm_q, buckets_q) and the window's keys and
// values from k and v through the keys' order; there is no self penalty, and
// a query whose window holds no key of its bucket gets a zero row and lse
// -inf. In the shared form q = k and the two orders are one.
template <int D, typename T, bool SEP>
__global__ __launch_bounds__(256) void attend_valu_kernel(const T* __restrict__ qsrc,
                                                          const T* __restrict__ ksrc,
                                                          const T* __restrict__ v,
                                                          const int32_t* __restrict__ buckets_q,
                                                          const int32_t* __restrict__ perm_q,
                                                          const int32_t* __restrict__ buckets_k,
                                                          const int32_t* __restrict__ perm_k,
                                                          Dims dm, int nqb,
                                                          float* __restrict__ o_sorted,
                                                          float* __restrict__ lse_sorted) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int QD = D / 4;   // features per lane
    constexpr int KB = 32;      // keys per LDS block
    constexpr int KS = D + 4;   // padded LDS row (floats)
    __shared__ __attribute__((aligned(16))) float ks[KB][KS];
    __shared__ __attribute__((aligned(16))) float vs[KB][KS];
    __shared__ int32_t kpos[KB], kbkt[KB];
    __shared__ float krn[KB];   // key scale: 1 / |x_j| with key normalisation, else 1
    const int64_t seg = block_y();
    if (seg >= dm.segs) return;
    const int64_t c = blockIdx.x / nqb;
    const int qb = (int)(blockIdx.x - c * nqb);
    const int tid = threadIdx.x, ql = tid >> 2, part = tid & 3;
    const int64_t L = dm.L, m = dm.m;
    const int64_t bh = seg / dm.nh;
    const int32_t* P = perm_k + seg * L;
    const int32_t* Bk = buckets_k + seg * L;
    const T* X = ksrc + bh * L * D;
    const T* V = v + bh * L * D;
    const int64_t qoff = (int64_t)qb * 64 + ql;   // query's place in its chunk
    const bool qlive = qoff < m;
    const int64_t s = c * m + (qlive ? qoff : 0); // its sorted slot (a real one when not live)
    const int64_t qpos = perm_q[seg * L + s];
    const int32_t qbkt = buckets_q[seg * L + qpos];
    float q[QD];
#pragma unroll
    for (int e = 0; e < QD; e += 4) {
        const f32x4 a = IO<T>::load4(qsrc + bh * L * D, qpos * D + part * QD + e);
        q[e] = a.x; q[e + 1] = a.y; q[e + 2] = a.z; q[e + 3] = a.w;
    }
    const float c2 = 1.4426950408889634f / sqrtf((float)D);   // log2(e) / sqrt(d)
    const float pen2 = kSelfPenalty * 1.4426950408889634f;
    float mx = -INFINITY, l = 0.f, acc[QD];
#pragma unroll
    for (int e = 0; e < QD; ++e) acc[e] = 0.f;
    const int64_t t0 = c > 0 ? (c - 1) * m : 0, t1 = (c + 1) * m;
    for (int64_t kb0 = t0; kb0 < t1; kb0 += KB) {
        const int nk = (int)min((int64_t)KB, t1 - kb0);
        __syncthreads();   // the previous block has been consumed
        if (tid < KB) {
            const int32_t p = tid < nk ? P[kb0 + tid] : -1;
            kpos[tid] = p;
            kbkt[tid] = p >= 0 ? Bk[p] : 0;
            krn[tid] = 1.f;
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
            if (dm.key_norm) {
                // the D/4 lanes of row j are consecutive and aligned in the wave
                float ss = a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
#pragma unroll
                for (int o = 1; o < D / 4; o <<= 1) ss += __shfl_xor(ss, o);
                if (k == 0) krn[j] = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
            }
        }
        __syncthreads();
        float sc[KB];
        float bmx = mx;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < QD; e += 4) {
                const f32x4 kk = *(const f32x4*)&ks[j][part * QD + e];
                dot = fmaf(q[e], kk.x, dot);
                dot = fmaf(q[e + 1], kk.y, dot);
                dot = fmaf(q[e + 2], kk.z, dot);
                dot = fmaf(q[e + 3], kk.w, dot);
            }
            dot += __shfl_xor(dot, 1);
            dot += __shfl_xor(dot, 2);
            const int32_t kp = kpos[j];
            const bool ok = j < nk && kbkt[j] == qbkt && (!dm.causal || kp <= qpos);
            const float s2 = dot * krn[j] * c2 - (!SEP && kp == qpos ? pen2 : 0.f);
            sc[j] = ok ? s2 : -INFINITY;
            bmx = fmaxf(bmx, sc[j]);
        }
        if (bmx == -INFINITY) continue;   // nothing valid yet (the same for a query's quad)
        const float rs = __builtin_amdgcn_exp2f(mx - bmx);   // 0 while mx = -inf
        l *= rs;
#pragma unroll
        for (int e = 0; e < QD; ++e) acc[e] *= rs;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            const float p = __builtin_amdgcn_exp2f(sc[j] - bmx);   // 0 where masked
            l += p;
#pragma unroll
            for (int e = 0; e < QD; e += 4) {
                const f32x4 vv = *(const f32x4*)&vs[j][part * QD + e];
                acc[e] = fmaf(p, vv.x, acc[e]);
                acc[e + 1] = fmaf(p, vv.y, acc[e + 1]);
                acc[e + 2] = fmaf(p, vv.z, acc[e + 2]);
                acc[e + 3] = fmaf(p, vv.w, acc[e + 3]);
            }
        }
        mx = bmx;
    }
    if (!qlive) return;
    // shared form: the query's own key is always in its window and valid, so
    // l > 0; separate queries and keys: l = 0 when no key counts
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    float* os = o_sorted + (seg * L + s) * D + part * QD;
#pragma unroll
    for (int e = 0; e < QD; e += 4)
        *(f32x4*)(os + e) = (f32x4){acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv,
                                    acc[e + 3] * inv};
    if (part == 0)
        lse_sorted[seg * L + s] = l > 0.f ? (mx + log2f(l)) * 0.6931471805599453f : -INFINITY;
}

// ---------------------------------------------------------------------------
// Matrix-core kernel (bf16 I/O, m = 64, d in {64, 128}).
//
// A workgroup (4 waves) walks a run of consecutive chunks of one (batch, head,
// round) segment. LDS holds a ring of two chunks: the qk rows (row-major,
// padded) and the v rows, keys indexed in ring order (slot * 64 + row) --
// the window of chunk c is simply both ring slots. The v rows feed the
// A operand of O^T = V^T P^T, which wants 8 consecutive keys of one feature
// per lane. At d = 128 the rows are stored as gathered (row-major) and two
// transposing LDS reads (ds_read_b64_tr_b16) take each operand from them; at
// d = 64 they are stored transposed (vt[feature][key]) and one 16-byte read
// does (measured: the transposing reads save the chunk pass 6 % at d = 128
// and cost it 3-4 % at d = 64).
// Each chunk's rows are gathered from HBM once, into registers, while the
// previous chunk(s) are being computed (kDepth chunks in flight; one measures
// as fast as two or three at 64K tokens), and serve as the look-back of the
// next. In the fused forward the sorted keys carry the bucket next to the
// position, so no bucket id is gathered.
//
// Wave w owns queries 16w..16w+15 of the chunk:
//   S^T = K Q^T   (v_mfma_f32_16x16x32_bf16; keys on rows, queries on lanes),
//                 only for 32-key blocks that can hold a valid key
//   mask, fp32 softmax in the exp2 domain
//   O^T = V^T P^T (P^T comes straight from the S^T registers: keys are
//                  assigned to S^T rows so each lane ends up holding 8
//                  consecutive keys, the B-operand layout)
// Lane layout of v_mfma_f32_16x16x32_bf16: A[m][k] in lane m%16 + 16*(k/8),
// element k%8; B[k][n] in lane n + 16*(k/8); D[m][n] in lane n + 16*(m/4),
// register m%4.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int kM = 64;            // chunk length of the matrix-core kernel
constexpr int kWin = 2 * kM;      // keys in a window
// Chunks per workgroup: 32 where the grid still holds at least eight
// workgroups per compute unit (2 % less chunk-pass time than 16 at 64K tokens
// x 8 heads x 8 rounds; 8 and 64 are slower), else 16 where it holds four,
// else 8. Same-box A/B of 16 against 8 (and 4) where 16 leaves two
// workgroups per compute unit, all one-round shapes: 64 x 1K 52.6 -> 43.3 us
// (47.0 with 4), 16 x 4K 54.4 -> 45.1, 4 x 16K 56.0 -> 46.9, 1 x 64K 57.3 ->
// 47.6; where 16 already gives four per unit (two rounds at 64 x 1K and
// 16 x 4K, 8 x 8 x 4K with four rounds) 8 is 1-4 % slower.
inline int attend_run_len(int64_t segs, int nchunks) {
    if (segs * ((nchunks + 31) / 32) >= 8 * 256) return 32;
    return segs * ((nchunks + 15) / 16) >= 4 * 256 ? 16 : 8;
}
// Chunks whose gathers are in flight behind the one computing: one measures
// as fast as two or three at 64K tokens and holds the fewest registers.
constexpr int kDepth = 1;
static_assert(kDepth >= 1 && kDepth <= 3, "key buffers hold four chunks");

template <int D>
struct alignas(16) AttendLds {
    static constexpr int KS = D + 8;       // padded row of qk (bf16 elements)
    static constexpr bool TRV = D == 128;  // v rows row-major, read transposed
    // TRV: v rows D + 16 elements apart, and 64 more after every 8 rows. A
    // transposing read takes 4 rows x 4 eight-byte pieces per 16 lanes: the
    // row step (8 banks) spreads them over 32 banks, and the extra 128 bytes
    // per 8 rows put the next 16 lanes (8 rows on) on the other 32.
    static constexpr int VRS = D + 16;
    static constexpr int vr_off(int r) { return r * VRS + (r >> 3) * 64; }
    // else: vt[feature][key], rows of VS elements
    static constexpr int VS = kWin + 8;
    uint16_t k[2][kM][KS];
    uint16_t vb[TRV ? kWin * VRS + (kWin / 8) * 64 : D * VS];
    int32_t pos[kWin];
    int32_t bkt[kWin];
    float rn[kWin];         // key scale (key normalisation): 1 / |x_j|
    int32_t nperm[4][kM];   // sorted keys of chunks waiting to be gathered
};

// KN (key normalisation): 0 off; 1 each key's 1 / |x| read from rn next to
// its position; 2 summed here from the pieces of the row being stored.
// SEP (separate queries and keys): the ring holds key rows from k through the
// keys' order (perm, buckets); each lane gathers its query row from q through
// the queries' order (perm_q, buckets_q) straight into its fragments, one
// chunk ahead; no self penalty, no causal block skip (the two orders differ),
// and a query without a key of its bucket gets a zero row and lse -inf.
template <int D, bool HALF, bool PACKED, int KN, bool SEP>
__global__ __launch_bounds__(256) void attend_mfma_kernel(const uint16_t* __restrict__ qk,
                                                          const uint16_t* __restrict__ v,
                                                          const int32_t* __restrict__ buckets,
                                                          const int32_t* __restrict__ perm,
                                                          Dims dm, int nruns, int run_len,
                                                          void* __restrict__ o_sorted,
                                                          const uint32_t* __restrict__ vmax,
                                                          const int direct,
                                                          float* __restrict__ lse_sorted,
                                                          const float* __restrict__ rn,
                                                          const uint16_t* __restrict__ qsep,
                                                          const int32_t* __restrict__ buckets_q,
                                                          const int32_t* __restrict__ perm_q) {
    constexpr int PIECES = D / 8;              // 16-byte pieces per row
    constexpr int QPT = kM * PIECES / 256;     // qk pieces per thread
    constexpr int QROWS = 256 / PIECES;        // rows covered per pass
    constexpr int KSTEPS = D / 32;
    constexpr int DT = D / 16;                 // output feature tiles
    __shared__ AttendLds<D> sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int64_t seg = blockIdx.x / nruns;
    const int run = blockIdx.x - (int)(seg * nruns);
    const int64_t L = dm.L;
    const int nchunks = dm.L / kM;
    const int c0 = run * run_len;
    const int c1 = min(c0 + run_len, nchunks);
    const int64_t bh = seg / dm.nh;
    const int32_t* P = perm + seg * L;
    const int32_t* Bk = buckets + seg * L;
    const uint16_t* X = qk + bh * L * D;
    const uint16_t* V = v + bh * L * D;
    const float c_log2 = 1.4426950408889634f / sqrtf((float)D);   // log2(e) / sqrt(d)
    const float pen2 = kSelfPenalty * 1.4426950408889634f;
    const float oscale = HALF && !direct ? o_scale(*vmax) : 1.0f;

    // sorted key of a slot: the position (plain perm) or bucket:position (packed)
    auto key_pos = [&](int32_t k) -> int { return PACKED ? (int)((uint32_t)k & kPackPosMask) : k; };

    // A operand of O^T = V^T P^T for key block kb (32 keys) and feature tile
    // dt: lane (g, r16) needs feature 16 dt + r16 of ring keys 32 kb + 8 g ..
    // + 7. In each 16-lane group, lane r16 addresses ring key 32 kb + 8 g +
    // 4 h + r16 / 4 at features 16 dt + 4 (r16 % 4) .. + 3; the transposing
    // read hands lane r16 feature 16 dt + r16 of those four keys, and h = 0, 1
    // give the 8 keys. Row 32 kb + 8 g + 4 h + r16 / 4 lies in 8-row block
    // 4 kb + g, so every address is this lane's base plus a constant.
    // (Without TRV: one 16-byte read of vt[16 dt + r16][32 kb + 8 g].)
    const uint16_t* vr_l = AttendLds<D>::TRV
        ? sm.vb + (8 * g + (r16 >> 2)) * AttendLds<D>::VRS + 64 * g + 4 * (r16 & 3)
        : sm.vb + r16 * AttendLds<D>::VS + 8 * g;
    auto v_frag = [&](int kb, int dt) -> u32x4 {
        if constexpr (AttendLds<D>::TRV) {
            const uint16_t* p = vr_l + 32 * kb * AttendLds<D>::VRS + 256 * kb + 16 * dt;
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
            const v4i16 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 4 * AttendLds<D>::VRS));
            const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
            return (u32x4){a.x, a.y, b.x, b.y};
        } else {
            return *(const u32x4*)(vr_l + 16 * dt * AttendLds<D>::VS + 32 * kb);
        }
    };

    // One chunk's rows in flight: gathered from HBM into registers (positions
    // from an LDS key buffer), parked in the LDS ring when the chunk's turn
    // comes. Two sets keep two chunks in flight behind the one computing.
    struct Rows {
        u32x4 q[QPT];
        u32x4 v[QPT];
        int32_t pos, bkt;   // position and bucket of row tid (threads < 64)
        float rn;           // and its 1 / |x| (KN == 1)
    };
    auto issue_rows = [&](Rows& rw, const int32_t* kl) {
#pragma unroll
        for (int j = 0; j < QPT; ++j) {
            const int row = tid / PIECES + QROWS * j;
            rw.q[j] = *(const u32x4*)(X + (int64_t)key_pos(kl[row]) * D + (tid % PIECES) * 8);
        }
        if constexpr (AttendLds<D>::TRV) {
#pragma unroll
            for (int j = 0; j < QPT; ++j) {
                const int row = tid / PIECES + QROWS * j;
                rw.v[j] = *(const u32x4*)(V + (int64_t)key_pos(kl[row]) * D + (tid % PIECES) * 8);
            }
        } else {
            // keys 2 pr and 2 pr + 1, features 8 ddg .. + 7
#pragma unroll
            for (int j = 0; j < QPT / 2; ++j) {
                const int pr = tid & 31, ddg = (tid >> 5) + 8 * j;
                rw.v[2 * j] = *(const u32x4*)(V + (int64_t)key_pos(kl[2 * pr]) * D + ddg * 8);
                rw.v[2 * j + 1] = *(const u32x4*)(V + (int64_t)key_pos(kl[2 * pr + 1]) * D + ddg * 8);
            }
        }
        if (tid < kM) {
            const int32_t k = kl[tid];
            rw.pos = key_pos(k);
            rw.bkt = PACKED ? (int32_t)((uint32_t)k >> kPackPosBits) : Bk[k];
            if constexpr (KN == 1) rw.rn = rn[bh * L + rw.pos];
        }
    };
    // registers -> ring slot; with KN == 2 each row's 1 / |x| is summed from
    // the pieces its PIECES consecutive lanes hold
    auto store_rows = [&](const Rows& rw, int slot) {
#pragma unroll
        for (int j = 0; j < QPT; ++j) {
            const int row = tid / PIECES + QROWS * j;
            *(u32x4*)&sm.k[slot][row][(tid % PIECES) * 8] = rw.q[j];
            if constexpr (KN == 2) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = __uint_as_float(rw.q[j][e] << 16);
                    const float hi = __uint_as_float(rw.q[j][e] & 0xFFFF0000u);
                    ss = fmaf(lo, lo, fmaf(hi, hi, ss));
                }
#pragma unroll
                for (int o = 1; o < PIECES; o <<= 1) ss += __shfl_xor(ss, o);
                if (tid % PIECES == 0) sm.rn[slot * kM + row] = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
            }
        }
        if constexpr (AttendLds<D>::TRV) {
#pragma unroll
            for (int j = 0; j < QPT; ++j) {
                const int row = tid / PIECES + QROWS * j;
                *(u32x4*)&sm.vb[AttendLds<D>::vr_off(slot * kM + row) + (tid % PIECES) * 8] = rw.v[j];
            }
        } else {
#pragma unroll
            for (int j = 0; j < QPT / 2; ++j) {
                const int pr = tid & 31, ddg = (tid >> 5) + 8 * j;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t lo = (rw.v[2 * j][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                    const uint32_t hi = (rw.v[2 * j + 1][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                    *(uint32_t*)&sm.vb[(ddg * 8 + e) * AttendLds<D>::VS + slot * kM + 2 * pr] =
                        lo | (hi << 16);
                }
            }
        }
        if (tid < kM) {
            sm.pos[slot * kM + tid] = rw.pos;
            sm.bkt[slot * kM + tid] = rw.bkt;
            if constexpr (KN == 1) sm.rn[slot * kM + tid] = rw.rn;
        }
    };

    // ---- separate queries: lane (g, r16) of wave w owns query row 16 w + r16
    // of each chunk; its fragments come from q, a chunk ahead, and the sorted
    // key of the row after that is fetched a further chunk ahead, so a row's
    // address never waits on a load issued in the same step.
    struct QRow {
        u32x4 f[KSTEPS];
        int32_t pos, bkt;
    };
    const int qrow_l = 16 * wave + r16;
    auto q_key = [&](int c) -> int32_t {
        return SEP ? perm_q[seg * L + (int64_t)c * kM + qrow_l] : 0;
    };
    auto issue_q = [&](QRow& qr, int32_t key) {
        qr.pos = key_pos(key);
        qr.bkt = PACKED ? (int32_t)((uint32_t)key >> kPackPosBits)
                        : buckets_q[seg * L + qr.pos];
        const uint16_t* row = qsep + (bh * L + qr.pos) * D + 8 * g;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qr.f[s] = *(const u32x4*)(row + 32 * s);
    };
    QRow qcur, qnext;
    int32_t qkey_next = 0;
    if constexpr (SEP) {
        issue_q(qcur, q_key(c0));
        if (c0 + 1 < c1) qkey_next = q_key(c0 + 1);
    }

    // ---- prologue: the look-back chunk c0-1 (or an empty slot) parked in its
    // ring slot; chunks c0 .. c0+DEPTH-1 in flight; the keys of c0+DEPTH in LDS.
    // Key buffers rotate over four slots (chunk & 3).
    Rows rw[kDepth];
    {
        const int slot = (c0 + 1) & 1;   // ring slot of chunk c0-1
        if (c0 > 0) {
            int32_t* kl = sm.nperm[(c0 - 1) & 3];
            if (tid < kM) kl[tid] = P[(int64_t)(c0 - 1) * kM + tid];
            __syncthreads();
            issue_rows(rw[0], kl);
            store_rows(rw[0], slot);
        } else {
            for (int k = tid; k < kM * AttendLds<D>::KS; k += 256) (&sm.k[slot][0][0])[k] = 0;
            if constexpr (AttendLds<D>::TRV) {
                for (int k = tid; k < kM * PIECES; k += 256)
                    *(u32x4*)&sm.vb[AttendLds<D>::vr_off(slot * kM + k / PIECES) + (k % PIECES) * 8] =
                        (u32x4){0u, 0u, 0u, 0u};
            } else {
                for (int k = tid; k < D * kM; k += 256)
                    sm.vb[(k / kM) * AttendLds<D>::VS + slot * kM + k % kM] = 0;
            }
            if (tid < kM) {
                sm.pos[slot * kM + tid] = 0;
                sm.bkt[slot * kM + tid] = -1;   // never equal to a bucket id
                sm.rn[slot * kM + tid] = 0.f;
            }
        }
        if (tid < kM)
            for (int c = c0; c <= c0 + kDepth && c < c1; ++c)
                sm.nperm[c & 3][tid] = P[(int64_t)c * kM + tid];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kDepth; ++j)
            if (c0 + j < c1) issue_rows(rw[j], sm.nperm[(c0 + j) & 3]);
    }

    auto step = [&](int c, Rows& rows) {
        const int cs = c & 1;
        store_rows(rows, cs);
        __syncthreads();
        // chunk c+DEPTH's rows go into the registers just parked, and the keys
        // of the chunk after it are fetched, while this chunk computes
        int32_t pf = 0;
        if (c + kDepth < c1) issue_rows(rows, sm.nperm[(c + kDepth) & 3]);
        if (c + kDepth + 1 < c1 && tid < kM) pf = P[(int64_t)(c + kDepth + 1) * kM + tid];
        if constexpr (SEP) {
            if (c + 1 < c1) issue_q(qnext, qkey_next);
            if (c + 2 < c1) qkey_next = q_key(c + 2);
        }

        // ---- which 32-key blocks can hold a valid key for any of this wave's
        // queries (wave-uniform): the block's bucket range must meet the
        // queries' (both are sorted within a chunk), and under causality an
        // own-chunk block that starts after the last query holds only later
        // positions of the same buckets.
        const int qrow = 16 * wave + r16;
        // lanes 0 and 15 hold the wave's first and last query rows
        const int qb_lo = SEP ? __builtin_amdgcn_readlane(qcur.bkt, 0)
                              : sm.bkt[cs * kM + 16 * wave];
        const int qb_hi = SEP ? __builtin_amdgcn_readlane(qcur.bkt, 15)
                              : sm.bkt[cs * kM + 16 * wave + 15];
        bool act[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int first = sm.bkt[32 * kb], last = sm.bkt[32 * kb + 31];
            bool a = first <= qb_hi && last >= qb_lo;
            if (!SEP && dm.causal && (kb >> 1) == cs && 32 * (kb & 1) > 16 * wave + 15)
                a = false;
            act[kb] = __builtin_amdgcn_readfirstlane((int)a) != 0;
        }

        // ---- S^T = K Q^T. Tile kt = 2*kb + h; A-row m holds key
        // 32*kb + 8*(m/4) + 4*h + m%4, so after both tiles of a block lane l
        // holds keys 32*kb + 8*(l/16) + e, e < 8: contiguous, ready to be the
        // B operand of the P^T V^T product.
        bf16x8 qf[KSTEPS];
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
            qf[s] = __builtin_bit_cast(
                bf16x8, SEP ? qcur.f[s] : *(const u32x4*)&sm.k[cs][qrow][32 * s + 8 * g]);
        const int qpos = SEP ? qcur.pos : sm.pos[cs * kM + qrow];
        const int qb = SEP ? qcur.bkt : sm.bkt[cs * kM + qrow];
        f32x4 st[8];
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            const int kb = kt >> 1, h = kt & 1;
            st[kt] = (f32x4){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            if (!act[kb]) continue;
            const int kw = 32 * kb + 8 * (r16 >> 2) + 4 * h + (r16 & 3);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, *(const u32x4*)&sm.k[kw >> 6][kw & 63][32 * s + 8 * g]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[s], acc, 0, 0, 0);
            }
            // mask (exp2 domain); register i is key 32*kb + 8*g + 4*h + i
            const i32x4 kbk = *(const i32x4*)&sm.bkt[32 * kb + 8 * g + 4 * h];
            const i32x4 kps = *(const i32x4*)&sm.pos[32 * kb + 8 * g + 4 * h];
            f32x4 krn = {1.f, 1.f, 1.f, 1.f};
            if constexpr (KN != 0) krn = *(const f32x4*)&sm.rn[32 * kb + 8 * g + 4 * h];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float s2 = acc[i] * krn[i] * c_log2 - (!SEP && kps[i] == qpos ? pen2 : 0.f);
                const bool ok = kbk[i] == qb && (!dm.causal || kps[i] <= qpos);
                s2 = ok ? s2 : -INFINITY;
                st[kt][i] = s2;
                mx = fmaxf(mx, s2);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // separate queries: a query without a key of its bucket keeps mx = -inf;
        // its exponentials are then taken against 0 (all of them are 0)
        const float mref = (SEP && mx == -INFINITY) ? 0.f : mx;

        // ---- P = exp2(s - max) as bf16; the P-weight sum that normalises O is
        // taken on the matrix cores from the same bf16 values (ones x P^T)
        float sum = 0.f;
        u32x4 pfrag[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (!act[kb]) continue;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float pr[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pr[i] = __builtin_amdgcn_exp2f(st[2 * kb + h][i] - mref);
                    sum += pr[i];
                }
                const bf16x2 w0 = {(__bf16)pr[0], (__bf16)pr[1]};
                const bf16x2 w1 = {(__bf16)pr[2], (__bf16)pr[3]};
                pfrag[kb][2 * h] = __builtin_bit_cast(uint32_t, w0);
                pfrag[kb][2 * h + 1] = __builtin_bit_cast(uint32_t, w1);
            }
        }
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);

        // ---- O^T = V^T P^T over the active blocks
        f32x4 oacc[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
        f32x4 osum = {0.f, 0.f, 0.f, 0.f};
        const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (!act[kb]) continue;
            const bf16x8 bfr = __builtin_bit_cast(bf16x8, pfrag[kb]);
            osum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ones), bfr,
                                                           osum, 0, 0, 0);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const u32x4 af = v_frag(kb, dt);
                oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af),
                                                                   bfr, oacc[dt], 0, 0, 0);
            }
        }
        const float sumr = osum[0];
        const int64_t slot = seg * L + (int64_t)c * kM + qrow;
        // by sorted slot (fp32), or -- in the fused forward -- already un-sorted:
        // row (b, h, position, round) in scaled fp16, so the combine streams
        const int64_t orow_idx = HALF ? (bh * L + qpos) * dm.nh + (seg - bh * dm.nh) : slot;
        if constexpr (HALF) {
            // (sumr = 0 only for a separate-keys query that found no key)
            const float inv = sumr > 0.f ? oscale / sumr : 0.f;
            // Lane (g, r16) holds features 16 dt + 4 g + i of its query. The
            // four lanes of a query swap pieces so that lane g stores features
            // 32 k + 8 g .. +7: each store then writes 64 contiguous bytes of
            // the row (half as many memory requests as 8-byte pieces).
            //
            // The row also carries the round's log-partition function (log2
            // domain): every 64-byte group of 32 features holds its 32 bits in
            // the lowest mantissa bit of each value -- word j of the group
            // (features 2j, 2j+1) holds bit j in its low half and bit 16 + j
            // in its high half. A separate lse array would be written 4 bytes
            // at a time at scattered positions, each store a partial memory
            // sector; this way the combine finds it in the row it reads
            // anyway. The cost is at most one fp16 ulp on each value.
            const uint32_t lb = __float_as_uint(mx + log2f(sum));
            uint32_t pat[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                pat[i] = ((lb >> (4 * g + i)) & 1u) | (((lb >> (16 + 4 * g + i)) & 1u) << 16);
            // With one round the row is the forward's output (weight 1): it is
            // written in bf16, unscaled, without the lse bits, into [B,H,L,d].
            u32x2 hv[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const f32x4 o = oacc[dt] * inv;
                if (direct) {
                    const bf16x4 h = {(__bf16)o.x, (__bf16)o.y, (__bf16)o.z, (__bf16)o.w};
                    hv[dt] = __builtin_bit_cast(u32x2, h);
                } else {
                    const f16x4 h = {(_Float16)o.x, (_Float16)o.y, (_Float16)o.z, (_Float16)o.w};
                    hv[dt] = __builtin_bit_cast(u32x2, h);
                }
            }
            // Lane (r16, g) holds A = features 32 k + 4 g .. + 3 (tile 2 k) and
            // B = 32 k + 16 + 4 g .. + 3 (tile 2 k + 1); lane g stores features
            // 32 k + 8 g .. + 7, i.e. A of lanes 2 g, 2 g + 1 (g < 2) or B of
            // lanes 2 g - 4, 2 g - 3. A lane swap between the two halves of
            // the wave (lanes 32 apart) and one between 16-lane rows do that
            // exchange on the vector unit.
            _Float16* orow = (_Float16*)o_sorted + orow_idx * D;
#pragma unroll
            for (int k = 0; k < DT / 2; ++k) {
                // A of rows 0, 1 with B of rows 0, 1 | A of rows 2, 3 with B of rows 2, 3
                const auto s0 = __builtin_amdgcn_permlane32_swap(hv[2 * k][0], hv[2 * k + 1][0], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(hv[2 * k][1], hv[2 * k + 1][1], false, false);
                // then rows pair up: lane g holds its 8 features' low 4 in [0], high 4 in [1]
                const auto t0 = __builtin_amdgcn_permlane16_swap(s0[0], s0[1], false, false);
                const auto t1 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
                const uint32_t w[4] = {t0[0], t1[0], t0[1], t1[1]};
                *(u32x4*)(orow + 32 * k + 8 * g) =
                    direct ? (u32x4){w[0], w[1], w[2], w[3]}
                           : (u32x4){(w[0] & 0xFFFEFFFEu) | pat[0], (w[1] & 0xFFFEFFFEu) | pat[1],
                                     (w[2] & 0xFFFEFFFEu) | pat[2], (w[3] & 0xFFFEFFFEu) | pat[3]};
            }
        } else {
            const float inv = sumr > 0.f ? 1.0f / sumr : 0.f;
            float* orow = (float*)o_sorted + slot * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) *(f32x4*)(orow + dt * 16 + 4 * g) = oacc[dt] * inv;
            if (g == 0) lse_sorted[slot] = (mx + log2f(sum)) * 0.6931471805599453f;   // -inf if empty
        }

        if (c + kDepth + 1 < c1 && tid < kM) sm.nperm[(c + kDepth + 1) & 3][tid] = pf;
        if constexpr (SEP) qcur = qnext;
        __syncthreads();
    };

    for (int c = c0; c < c1; c += kDepth) {
#pragma unroll
        for (int j = 0; j < kDepth; ++j)
            if (c + j < c1) step(c + j, rw[j]);
    }
}

template <typename T, bool SEP>
static void launch_valu(const T* qsrc, const T* ksrc, const T* v, const int32_t* bq,
                        const int32_t* pq, const int32_t* bk, const int32_t* pk, const Dims& d,
                        float* o, float* lse, hipStream_t st) {
    const int nqb = (d.m + 63) / 64;   // 64-query blocks per chunk
    const dim3 grid = grid_split((unsigned)((int64_t)(d.L / d.m) * nqb), d.segs);
    if (d.d == 64)
        attend_valu_kernel<64, T, SEP><<<grid, 256, 0, st>>>(qsrc, ksrc, v, bq, pq, bk, pk, d,
                                                             nqb, o, lse);
    else
        attend_valu_kernel<128, T, SEP><<<grid, 256, 0, st>>>(qsrc, ksrc, v, bq, pq, bk, pk, d,
                                                              nqb, o, lse);
}

template <typename T>
static void launch_valu_any(const void* qk, const void* v, const int32_t* buckets,
                            const int32_t* perm, const SepQK* sep, const Dims& d, float* o,
                            float* lse, hipStream_t st) {
    const T* k = (const T*)qk;
    if (sep)
        launch_valu<T, true>((const T*)sep->q, k, (const T*)v, sep->buckets_q, sep->perm_q,
                             buckets, perm, d, o, lse, st);
    else
        launch_valu<T, false>(k, k, (const T*)v, buckets, perm, buckets, perm, d, o, lse, st);
}

hipError_t launch_attend(const void* qk, const void* v, const int32_t* buckets,
                         const int32_t* perm, const Dims& d, const OSorted& o, float* lse_sorted,
                         hipStream_t st, hipEvent_t* ev, int* nev, const char** names,
                         bool packed, const float* rn, const SepQK* sep) {
    if (packed && !(o.half && d.dtype == LSH_BF16 && d.m == kM)) return hipErrorInvalidValue;
    if (o.direct && !(o.half && d.nh == 1 && d.dtype == LSH_BF16 && d.m == kM && !sep))
        return hipErrorInvalidValue;
    if (sep && d.key_norm) return hipErrorInvalidValue;
    if (d.dtype == LSH_BF16 && d.m == kM) {
        const int nchunks = d.L / kM;
        const int run_len = attend_run_len(d.segs, nchunks);
        const int nruns = (nchunks + run_len - 1) / run_len;
        const unsigned grid = (unsigned)(d.segs * nruns);
        const uint16_t* x = (const uint16_t*)qk;
        const uint16_t* vv = (const uint16_t*)v;
        const uint16_t* qs = sep ? (const uint16_t*)sep->q : nullptr;
        const int32_t* bq = sep ? sep->buckets_q : nullptr;
        const int32_t* pq = sep ? sep->perm_q : nullptr;
#define LSH_ATTEND_ARGS(VM, RN) \
    x, vv, buckets, perm, d, nruns, run_len, o.ptr, VM, (int)o.direct, lse_sorted, RN, qs, bq, pq
#define LSH_ATTEND_LAUNCH(DD, HH, PP, VM)                                                      \
    (sep ? attend_mfma_kernel<DD, HH, PP, 0, true><<<grid, 256, 0, st>>>(                      \
               LSH_ATTEND_ARGS(VM, nullptr))                                                   \
     : !d.key_norm ? attend_mfma_kernel<DD, HH, PP, 0, false><<<grid, 256, 0, st>>>(           \
                         LSH_ATTEND_ARGS(VM, nullptr))                                         \
     : rn ? attend_mfma_kernel<DD, HH, PP, 1, false><<<grid, 256, 0, st>>>(                    \
                LSH_ATTEND_ARGS(VM, rn))                                                       \
          : attend_mfma_kernel<DD, HH, PP, 2, false><<<grid, 256, 0, st>>>(                    \
                LSH_ATTEND_ARGS(VM, nullptr)))
        if (o.half && packed) {
            if (d.d == 64) LSH_ATTEND_LAUNCH(64, true, true, o.vmax);
            else LSH_ATTEND_LAUNCH(128, true, true, o.vmax);
        } else if (o.half) {
            if (d.d == 64) LSH_ATTEND_LAUNCH(64, true, false, o.vmax);
            else LSH_ATTEND_LAUNCH(128, true, false, o.vmax);
        } else {
            if (d.d == 64) LSH_ATTEND_LAUNCH(64, false, false, nullptr);
            else LSH_ATTEND_LAUNCH(128, false, false, nullptr);
        }
#undef LSH_ATTEND_LAUNCH
#undef LSH_ATTEND_ARGS
        return mark(st, ev, nev, names, "attend_mfma");
    }
    float* of = (float*)o.ptr;
    if (d.dtype == LSH_BF16)
        launch_valu_any<uint16_t>(qk, v, buckets, perm, sep, d, of, lse_sorted, st);
    else
        launch_valu_any<float>(qk, v, buckets, perm, sep, d, of, lse_sorted, st);
    return mark(st, ev, nev, names, "attend_fp32");
}

}  // namespace lsh
