// lsh_internal.h -- shared declarations of the gfx950 LSH-attention kernels.
//
// Host launchers are defined next to their kernels (lsh_hash.hip, lsh_sort.hip,
// lsh_attend.hip, lsh_combine.hip) and called by the C ABI in lsh_api.hip.
// Every launcher enqueues on the given stream and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsh_attn.h"

namespace lsh {

constexpr int kWave = 64;
constexpr float kSelfPenalty = 1.0e5f;   // subtracted from a query's score against itself

// Device-side problem description (plain values, passed by value to kernels).
struct Dims {
    int32_t B, H, L, d;
    int32_t nb, nh, m, causal;
    int32_t dtype;
    int32_t key_norm;   // keys as unit vectors in the scores (LSH_KEY_NORM)
    int32_t per_head_r; // R is [H, nh, d, nb/2]: each head its own rotations
    int32_t nr;         // rounds of R: nh, or H*nh with per-head rotations; head h's
                        // round r is R round h*nh + r (a "virtual round")
    int64_t T;        // B*H*L token-heads
    int64_t segs;     // B*H*nh (batch, head, round) segments
};

inline Dims make_dims(const lsh_shape_t& s) {
    Dims d{};
    d.B = s.B; d.H = s.H; d.L = s.L; d.d = s.d;
    d.nb = s.n_buckets; d.nh = s.n_hashes; d.m = s.chunk_len; d.causal = s.causal;
    d.dtype = s.dtype;
    d.key_norm = (s.flags & LSH_KEY_NORM) ? 1 : 0;
    d.per_head_r = (s.flags & LSH_PER_HEAD_R) ? 1 : 0;
    d.nr = d.per_head_r ? s.H * s.n_hashes : s.n_hashes;
    d.T = (int64_t)s.B * s.H * s.L;
    d.segs = (int64_t)s.B * s.H * s.n_hashes;
    return d;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Grids of nx x ny workgroups whose second count can pass the 65535 a grid
// dimension holds (segments B*H*n_hashes, rotation rounds, row tiles): ny is
// split over y and z, block_y() recovers the index, and the few blocks past
// ny return before doing anything.
constexpr int64_t kGridYZ = 65535;
inline dim3 grid_split(unsigned nx, int64_t ny) {
    const int64_t y = ny < kGridYZ ? (ny > 0 ? ny : 1) : kGridYZ;
    return dim3(nx, (unsigned)y, (unsigned)((ny + y - 1) / y));
}
__device__ __forceinline__ int64_t block_y() {
    return (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
}

// ---------------------------------------------------------------- hash stage
// Column tile of the matrix-core hash pass: 32 projection columns.
constexpr int kHashColTile = 32;

inline int hash_ntiles(const Dims& d) { return (d.nb / 2 + kHashColTile - 1) / kHashColTile; }

// One entry of the re-decision queue written by the fast hash pass.
//   item : flat index into buckets [B,H,nh,L]
//   a, b : the two candidate columns (mode 0) -- unused for mode 1
//   mode : 0 = decide between columns a and b, 1 = scan every column
struct RefineItem {
    int32_t item, a, b, mode;
};

// The queue is cut into fixed regions, one per wave of the fast pass, so a
// wave appends without any atomic: two-candidate items fill its region from
// the front, full scans from the back, and the wave stores the two counts
// (rcount[2 * region], rcount[2 * region + 1]) when it ends. Capacity covers
// T rounded up to kQueuePad tokens, every round -- with per-head rotations,
// where a workgroup's tokens stay inside one (batch, head), every L is
// rounded up (a sum of round-ups is at least the round-up of the sum).
constexpr int kQueuePad = 256;
inline int64_t queue_tokens(const Dims& d) {
    if (d.per_head_r) return (int64_t)d.B * d.H * ((d.L + kQueuePad - 1) / kQueuePad * kQueuePad);
    return (d.T + kQueuePad - 1) / kQueuePad * kQueuePad;
}

// R round used by round r of (batch, head) bh.
__host__ __device__ inline int r_round(const Dims& d, int64_t bh, int r) {
    return d.per_head_r ? (int)(bh % d.H) * d.nh + r : r;
}

struct HashWorkspace {
    int32_t* counter;     // [0]: items re-decided (the public count)
    uint32_t* vmax;       // max|v| (bf16 bits) when the fast pass is asked to fold it in
    // Per (bound, R round, 32-column tile) bounds, [3][nr][ntiles], each rounded
    // up; a round's bound is the largest over its tiles. With R_s = R * 2^e_r,
    // e_r the power of two that brings max|R| of round r into [2^14, 2^15):
    //   bound 0  largest column 2-norm of R
    //   bound 1  largest column 2-norm of R_s
    //   bound 2  largest column 2-norm of R_s - fp16(R_s), plus the fp16
    //            subnormal elements a matrix core may flush
    float* tnorm;
    uint16_t* rfrag;      // fp16(R_s) in matrix-core fragment order
    float* rt;            // R transposed to [nr][ntiles*32][d], fp32
    RefineItem* queue;    // [queue_tokens * nh]
    int32_t* rcount;      // [2 * queue_tokens * nh / 64]: per-region counts
    // Full-scan items regrouped by R round for the scan pass: per R round r,
    // scount[r] items, slist[r * queue_tokens + i] their flat bucket index and
    // sbest[r * queue_tokens + i] the best packed key found so far.
    int32_t* scount;      // [nr]
    int32_t* slist;       // [nr * queue_tokens]
    uint64_t* sbest;      // [nr * queue_tokens]
};
size_t hash_workspace_bytes(const Dims& d);
HashWorkspace carve_hash_workspace(void* ws, const Dims& d);

// v_for_max (bf16 values, or null): also fold max|v| into w.vmax during the
// matrix-core pass (only bf16 inputs take that pass).
hipError_t launch_hash(const void* qk, const float* R, const Dims& d, int32_t* buckets,
                       const HashWorkspace& w, hipStream_t st, hipEvent_t* ev, int* nev,
                       const char** names, const void* v_for_max = nullptr);

// ---------------------------------------------------------------- sort stage
constexpr int kSortTile = 4096;          // elements per sort tile (one workgroup)
constexpr int kSortWaves = 4;            // waves per sort workgroup
constexpr int kMaxBuckets = 4096;
constexpr int kMaxHashes = 4096;

inline int64_t sort_ntiles(const Dims& d) { return (d.L + kSortTile - 1) / kSortTile; }
size_t sort_workspace_bytes(const Dims& d);

// Size of the static scratch behind lsh_sort_noalloc, and its device address
// on the current device (looked up once per device).
constexpr size_t kSortScratchBytes = (size_t)16 << 20;
hipError_t sort_scratch(void** ptr);

// Packed sorted keys: inside the fused forward the sort can store, per slot,
// (bucket << kPackPosBits) | position instead of the plain position, so the
// chunk pass reads both from one coalesced word; no inverse is written then.
constexpr int kPackPosBits = 20;
constexpr uint32_t kPackPosMask = (1u << kPackPosBits) - 1u;
inline bool packed_sort_keys(const Dims& d) { return d.L <= (1 << kPackPosBits); }

hipError_t launch_sort(const int32_t* buckets, const Dims& d, int32_t* perm, int32_t* inv,
                       void* ws, hipStream_t st, hipEvent_t* ev, int* nev, const char** names,
                       bool packed = false);

// ------------------------------------------------------------ attend stage
// Per-round outputs: float32 by sorted slot ([B,H,nh,L,d], with lse
// [B,H,nh,L]) for the staged entry points; inside the fused forward on the
// matrix-core path ("half"), fp16 multiplied by a power of two derived from
// max|v| (o_scale), so no value can overflow, stored already un-sorted by
// position ([B,H,L,nh,d]); each 64-byte group of a row then carries that
// round's lse (log2 domain) in its values' lowest mantissa bits and no lse
// array is written.
struct OSorted {
    void* ptr;                  // float* or _Float16*
    bool half;                  // fp16 by position
    const uint32_t* vmax;       // bf16 bit pattern of max|v| (used when half)
    bool direct = false;        // half with one round: ptr is the bf16 output [B,H,L,d]
};

// True when the fused forward can keep o_sorted in scaled fp16.
inline bool compact_o_sorted(const Dims& d) { return d.dtype == LSH_BF16 && d.m == 64; }

// Separate queries and keys: the queries' tensor and sorted order. The
// attend launcher's qk / buckets / perm then describe the keys.
struct SepQK {
    const void* q;
    const int32_t* buckets_q;   // [B,H,nh,L] by position (read when keys are not packed)
    const int32_t* perm_q;      // [B,H,nh,L] sorted (packed like perm when packed)
};

// packed: perm holds packed sorted keys (buckets is then not read); only
// the fp16 by-position form takes them.
// With d.key_norm, rn holds 1 / |qk| per token (launch_key_rnorm); when it is
// null the kernels sum each staged row's squares themselves.
// sep (or null): separate queries and keys -- qk, buckets and perm are the
// keys', sep the queries'; outputs by query slot (or query position).
hipError_t launch_attend(const void* qk, const void* v, const int32_t* buckets,
                         const int32_t* perm, const Dims& d, const OSorted& o, float* lse_sorted,
                         hipStream_t st, hipEvent_t* ev, int* nev, const char** names,
                         bool packed = false, const float* rn = nullptr,
                         const SepQK* sep = nullptr);

// ----------------------------------------------------- feed-forward
// out = relu(x W1^T + b1) W2^T + b2 over `rows` rows, chunk_rows at a time;
// inter holds one chunk's intermediate (min(chunk_rows, rows) * d_ff elements).
hipError_t launch_ffn(const void* x, const void* w1, const void* b1, const void* w2,
                      const void* b2, int64_t rows, int d_model, int d_ff, int chunk_rows,
                      bool bf16, void* out, void* inter, hipStream_t st);

// ----------------------------------------------------- key normalisation
// rn[t] = 1 / |qk[t]| (0 for the zero vector), float32, one per token-head.
hipError_t launch_key_rnorm(const void* qk, const Dims& d, float* rn, hipStream_t st);

// ----------------------------------------------------------- combine stage
// z (or null): per token [B,H,L], the natural-log partition function over
// every round, logsumexp_r lse_r -- what the backward needs besides the sort.
hipError_t launch_combine(const OSorted& o, const float* lse_sorted, const int32_t* inv,
                          const Dims& d, void* out, hipStream_t st, hipEvent_t* ev, int* nev,
                          const char** names, float* z = nullptr);

// ----------------------------------------------------- input projections
// qk, v [B,H,L,d] from x [B,L,d_model] and weights [H*d, d_model].
hipError_t launch_project(const void* x, const void* w_qk, const void* w_v, const Dims& d,
                          int d_model, void* qk, void* v, hipStream_t st);

// --------------------------------------------------------------- backward
// Gradients from the saved sort (perm: packed keys when `packed`, else
// positions with bucket ids by position in `buckets`) and Z per token.
struct BwdArgs {
    const void* qk;
    const void* v;
    const void* out;
    const void* dout;
    const int32_t* perm;      // [B,H,nh,L]
    const int32_t* buckets;   // [B,H,nh,L] by position
    const float* z;           // [B,H,L] natural-log total partition function
    float* Dv;                // [B,H,L] scratch: dout . out
    const float* rn;          // [B,H,L] 1 / |qk| (key normalisation), else null
    float* dx_r;              // [B,H,L,nh,d] scratch: per-round dq + dk
    float* dv_r;              // [B,H,L,nh,d] scratch: per-round dv
    void* dqk;                // [B,H,L,d] out
    void* dv;                 // [B,H,L,d] out
};
hipError_t launch_backward(const BwdArgs& a, const Dims& d, bool packed, hipStream_t st);

// Power of two s with max|v| * s <= 2^14: fp16 then holds every |o| <= max|v|.
__device__ __forceinline__ float o_scale(uint32_t vmax_bf16) {
    const uint32_t bits = (vmax_bf16 & 0x7FFFu) << 16;
    if (bits == 0) return 1.0f;
    const int e = (int)(bits >> 23) - 127;   // max|v| < 2^(e+1)
    int k = 14 - (e + 1);
    k = k < -126 ? -126 : (k > 100 ? 100 : k);
    return __uint_as_float((uint32_t)(k + 127) << 23);
}

// Records a timing event after a kernel when the caller asked for timing.
inline hipError_t mark(hipStream_t st, hipEvent_t* ev, int* nev, const char** names,
                       const char* name) {
    if (!ev) return hipSuccess;
    if (names) names[*nev] = name;
    hipError_t e = hipEventRecord(ev[*nev + 1], st);
    ++*nev;
    return e;
}

// ------------------------------------------------------------ device helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// float -> bf16, round to nearest even (finite inputs; NaN stays NaN)
// Round to nearest even (the hardware conversion, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <typename T>
struct IO;
typedef float io_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t io_u32x2 __attribute__((ext_vector_type(2)));
template <>
struct IO<float> {
    __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
    // four consecutive elements; p + i must be 16-byte aligned
    __device__ __forceinline__ static io_f32x4 load4(const float* p, int64_t i) {
        return *(const io_f32x4*)(p + i);
    }
    __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <>
struct IO<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t* p, int64_t i) {
        return bf16_to_f32(p[i]);
    }
    // four consecutive elements; p + i must be 8-byte aligned
    __device__ __forceinline__ static io_f32x4 load4(const uint16_t* p, int64_t i) {
        const io_u32x2 w = *(const io_u32x2*)(p + i);
        return (io_f32x4){__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                          __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
    }
    __device__ __forceinline__ static void store(uint16_t* p, int64_t i, float v) {
        p[i] = f32_to_bf16(v);
    }
};

}  // namespace lsh
