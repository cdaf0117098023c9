// lsh_api.hip -- the C ABI declared in include/lsh_attn.h: host-side argument
// checks, workspace layout and launch order. Nothing here touches the device
// before the arguments have been validated, and loading the library does not
// initialise HIP.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include <initializer_list>

#include "lsh_internal.h"

using namespace lsh;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

// Test hook (lsh_debug_fail_launch): launcher statuses left before one is
// reported as failed; 0 = off. The launches themselves are never touched.
thread_local int g_fail_in = 0;
thread_local bool g_injected = false;

hipError_t checked(hipError_t e) {
    if (e == hipSuccess && g_fail_in > 0 && --g_fail_in == 0) {
        g_injected = true;
        return hipErrorLaunchFailure;
    }
    return e;
}

int hip_fail(hipError_t e, const char* where) {
    const bool inj = g_injected;
    g_injected = false;
    return fail(LSH_ERR_HIP, "%s: %s%s", where, hipGetErrorString(e),
                inj ? " (injected by lsh_debug_fail_launch)" : "");
}

int validate(const lsh_shape_t* s) {
    if (!s) return fail(LSH_ERR_ARG, "shape is NULL");
    if (s->B < 0 || s->H < 0 || s->L < 0)
        return fail(LSH_ERR_ARG, "negative B/H/L (%d, %d, %d)", s->B, s->H, s->L);
    if (s->d < 1) return fail(LSH_ERR_ARG, "d must be positive (got %d)", s->d);
    if (s->n_buckets < 2 || (s->n_buckets % 2) != 0)
        return fail(LSH_ERR_ARG, "n_buckets must be even and >= 2 (got %d)", s->n_buckets);
    if (s->n_buckets > kMaxBuckets)
        return fail(LSH_ERR_ARG, "n_buckets must be at most %d (got %d)", kMaxBuckets,
                    s->n_buckets);
    if (s->n_hashes < 1 || s->n_hashes > kMaxHashes)
        return fail(LSH_ERR_ARG, "n_hashes must be in [1, %d] (got %d)", kMaxHashes, s->n_hashes);
    if (s->chunk_len < 1) return fail(LSH_ERR_ARG, "chunk_len must be >= 1 (got %d)", s->chunk_len);
    if (s->L % s->chunk_len != 0)
        return fail(LSH_ERR_ARG, "L (%d) must be a multiple of chunk_len (%d)", s->L, s->chunk_len);
    if (s->causal != 0 && s->causal != 1)
        return fail(LSH_ERR_ARG, "causal must be 0 or 1 (got %d)", s->causal);
    if (s->dtype != LSH_F32 && s->dtype != LSH_BF16)
        return fail(LSH_ERR_ARG, "dtype must be LSH_F32 or LSH_BF16 (got %d)", s->dtype);
    if (s->flags & ~(LSH_KEY_NORM | LSH_PER_HEAD_R))
        return fail(LSH_ERR_ARG, "unknown flags 0x%x (only LSH_KEY_NORM, LSH_PER_HEAD_R)",
                    (unsigned)s->flags);
    if ((int64_t)s->B * s->H * s->n_hashes * s->L >= ((int64_t)1 << 31))
        return fail(LSH_ERR_ARG, "B*H*n_hashes*L must stay below 2^31");
    if (s->d != 64 && s->d != 128)
        return fail(LSH_ERR_ARG, "head size d must be 64 or 128 (got %d)", s->d);
    return LSH_OK;
}

bool empty(const lsh_shape_t* s) { return s->B == 0 || s->H == 0 || s->L == 0; }

// Non-zero when any of the pointers is not 16-byte aligned (NULLs pass).
int misaligned(std::initializer_list<const void*> ptrs) {
    for (const void* p : ptrs)
        if (reinterpret_cast<uintptr_t>(p) & 15u) return 1;
    return 0;
}

struct FwdLayout {
    size_t hash, sort, buckets, perm, inv, lse, o, rn, bk, pk, ik, total;
};

// sep: separate queries and keys -- the keys' bucket ids and sorted order
// follow (and their inverse when the sort cannot pack its keys).
FwdLayout fwd_layout(const Dims& d, bool sep = false) {
    FwdLayout f;
    const size_t n = (size_t)d.segs * d.L;
    size_t off = 0;
    f.hash = off;
    off += align_up(hash_workspace_bytes(d), 256);
    f.sort = off;
    off += align_up(sort_workspace_bytes(d), 256);
    f.buckets = off;
    off += align_up(sizeof(int32_t) * n, 256);
    f.perm = off;
    off += align_up(sizeof(int32_t) * n, 256);
    // The fp16 by-position rows carry their own lse and, with packed sort
    // keys, need no inverse permutation: those regions are then empty.
    const bool compact = compact_o_sorted(d);
    const bool packed = compact && packed_sort_keys(d);
    f.inv = off;
    off += packed ? 0 : align_up(sizeof(int32_t) * n, 256);
    f.lse = off;
    off += compact ? 0 : align_up(sizeof(float) * n, 256);
    f.o = off;
    off += align_up((compact ? 2 : sizeof(float)) * n * d.d, 256);
    // key normalisation: 1 / |qk| per token, computed once per call
    f.rn = off;
    off += d.key_norm ? align_up(sizeof(float) * (size_t)d.T, 256) : 0;
    f.bk = off;
    off += sep ? align_up(sizeof(int32_t) * n, 256) : 0;
    f.pk = off;
    off += sep ? align_up(sizeof(int32_t) * n, 256) : 0;
    f.ik = off;
    off += sep && !packed ? align_up(sizeof(int32_t) * n, 256) : 0;
    f.total = off;
    return f;
}

int check_ws(const char* stage, const Dims& d, void* ws, size_t ws_bytes, size_t need) {
    (void)d;
    if (!ws) return fail(LSH_ERR_WORKSPACE, "%s: workspace is NULL", stage);
    if (misaligned({ws})) return fail(LSH_ERR_ARG, "%s: workspace must be 16-byte aligned", stage);
    if (ws_bytes < need)
        return fail(LSH_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", stage, ws_bytes,
                    need);
    return LSH_OK;
}

// The state a training forward leaves for the backward: bucket ids by
// position, the sorted keys (packed when the fused path packs them) and Z.
struct StateLayout {
    size_t buckets, perm, z, total;
};

StateLayout state_layout(const Dims& d) {
    StateLayout s;
    const size_t n = (size_t)d.segs * d.L;
    s.buckets = 0;
    s.perm = align_up(sizeof(int32_t) * n, 256);
    s.z = s.perm + align_up(sizeof(int32_t) * n, 256);
    s.total = s.z + align_up(sizeof(float) * (size_t)d.T, 256);
    return s;
}

bool fused_packed(const Dims& d) { return compact_o_sorted(d) && packed_sort_keys(d); }

struct BwdLayout {
    size_t dvec, dx, dv, rn, total;
};

BwdLayout bwd_layout(const Dims& d) {
    BwdLayout b;
    const size_t rows = (size_t)d.T * d.nh * d.d;
    b.dvec = 0;
    b.dx = align_up(sizeof(float) * (size_t)d.T, 256);
    b.dv = b.dx + align_up(sizeof(float) * rows, 256);
    b.rn = b.dv + align_up(sizeof(float) * rows, 256);
    b.total = b.rn + (d.key_norm ? align_up(sizeof(float) * (size_t)d.T, 256) : 0);
    return b;
}

// state (or null): where the sort and Z go for a later backward.
int run_fwd(const void* qk, const void* v, const float* R, const lsh_shape_t* shape, void* out,
            void* ws, size_t ws_bytes, hipStream_t st, hipEvent_t* ev, int* nev,
            const char** names, void* state = nullptr) {
    const Dims d = make_dims(*shape);
    const FwdLayout f = fwd_layout(d);
    int rc = check_ws("lsh_attention_fwd", d, ws, ws_bytes, f.total);
    if (rc) return rc;
    char* base = (char*)ws;
    int32_t* buckets = (int32_t*)(base + f.buckets);
    int32_t* perm = (int32_t*)(base + f.perm);
    float* z = nullptr;
    if (state) {
        const StateLayout sl = state_layout(d);
        buckets = (int32_t*)((char*)state + sl.buckets);
        perm = (int32_t*)((char*)state + sl.perm);
        z = (float*)((char*)state + sl.z);
    }
    int32_t* inv = (int32_t*)(base + f.inv);
    float* lse = (float*)(base + f.lse);
    const HashWorkspace hw = carve_hash_workspace(base + f.hash, d);
    // the compact path (bf16 I/O) takes the matrix-core hash, which also
    // produces max|v| for the scale of the fp16 per-round outputs. With one
    // round that round's output is the forward's (weight 1): the chunk pass
    // writes it in bf16 straight into out and no combine runs -- except in
    // the training forward, whose combine also writes Z.
    const bool compact = compact_o_sorted(d);
    const bool direct = compact && d.nh == 1 && !z;
    const OSorted o{direct ? out : base + f.o, compact, hw.vmax, direct};
    hipError_t e;
    if ((e = checked(launch_hash(qk, R, d, buckets, hw, st, ev, nev, names,
                                 compact && !direct ? v : nullptr))) != hipSuccess)
        return hip_fail(e, "hash");
    // the fp16 by-position form un-sorts in the chunk pass, so the sort can
    // hand it packed keys and skip the inverse permutation
    const bool packed = compact && packed_sort_keys(d);
    if ((e = checked(launch_sort(buckets, d, perm, inv, base + f.sort, st, ev, nev, names,
                                 packed))) != hipSuccess)
        return hip_fail(e, "sort");
    float* rn = nullptr;
    if (d.key_norm) {
        rn = (float*)(base + f.rn);
        if ((e = checked(launch_key_rnorm(qk, d, rn, st))) != hipSuccess ||
            (e = mark(st, ev, nev, names, "key_rnorm")) != hipSuccess)
            return hip_fail(e, "key_rnorm");
    }
    if ((e = checked(launch_attend(qk, v, buckets, perm, d, o, lse, st, ev, nev, names, packed,
                                   rn))) != hipSuccess)
        return hip_fail(e, "chunk_attend");
    if (!direct &&
        (e = checked(launch_combine(o, lse, inv, d, out, st, ev, nev, names, z))) != hipSuccess)
        return hip_fail(e, "unsort_combine");
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "launch");
    return LSH_OK;
}

// Separate queries and keys: both hashed with the same R and sorted on their
// own, then the chunk pass with the keys' order in the ring and the queries'
// order on the query side, then the combine through the queries' order.
int run_fwd_qk(const void* q, const void* k, const void* v, const float* R,
               const lsh_shape_t* shape, void* out, void* ws, size_t ws_bytes, hipStream_t st) {
    const Dims d = make_dims(*shape);
    const FwdLayout f = fwd_layout(d, true);
    int rc = check_ws("lsh_attention_fwd_qk", d, ws, ws_bytes, f.total);
    if (rc) return rc;
    char* base = (char*)ws;
    int32_t* bq = (int32_t*)(base + f.buckets);
    int32_t* pq = (int32_t*)(base + f.perm);
    int32_t* iq = (int32_t*)(base + f.inv);
    int32_t* bk = (int32_t*)(base + f.bk);
    int32_t* pk = (int32_t*)(base + f.pk);
    int32_t* ik = (int32_t*)(base + f.ik);
    float* lse = (float*)(base + f.lse);
    const HashWorkspace hw = carve_hash_workspace(base + f.hash, d);
    const bool compact = compact_o_sorted(d);
    const bool packed = compact && packed_sort_keys(d);
    const OSorted o{base + f.o, compact, hw.vmax};
    hipError_t e;
    // the keys' pass folds max|v| (each hash pass clears it first)
    if ((e = checked(launch_hash(q, R, d, bq, hw, st, nullptr, nullptr, nullptr))) !=
            hipSuccess ||
        (e = checked(launch_hash(k, R, d, bk, hw, st, nullptr, nullptr, nullptr,
                                 compact ? v : nullptr))) != hipSuccess)
        return hip_fail(e, "hash");
    if ((e = checked(launch_sort(bq, d, pq, iq, base + f.sort, st, nullptr, nullptr, nullptr,
                                 packed))) != hipSuccess ||
        (e = checked(launch_sort(bk, d, pk, ik, base + f.sort, st, nullptr, nullptr, nullptr,
                                 packed))) != hipSuccess)
        return hip_fail(e, "sort");
    const SepQK sep{q, bq, pq};
    if ((e = checked(launch_attend(k, v, bk, pk, d, o, lse, st, nullptr, nullptr, nullptr,
                                   packed, nullptr, &sep))) != hipSuccess)
        return hip_fail(e, "chunk_attend");
    if ((e = checked(launch_combine(o, lse, iq, d, out, st, nullptr, nullptr, nullptr))) !=
        hipSuccess)
        return hip_fail(e, "unsort_combine");
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "launch");
    return LSH_OK;
}

// One projected tensor ([B,H,L,d] in the I/O dtype), rounded up so the next
// region stays 256-byte aligned.
size_t projected_bytes(const Dims& d) {
    return align_up((size_t)d.T * d.d * (d.dtype == LSH_BF16 ? 2 : 4), 256);
}

// Bytes of one chunk's intermediate of the chunked feed-forward.
int ffn_workspace(int64_t rows, int32_t d_ff, int32_t chunk_rows, int32_t dtype, size_t* bytes) {
    if (rows < 0 || d_ff < 8 || d_ff % 8 != 0 || chunk_rows < 1 ||
        (dtype != LSH_F32 && dtype != LSH_BF16))
        return fail(LSH_ERR_ARG,
                    "lsh_ffn: rows >= 0, d_ff a positive multiple of 8, chunk_rows >= 1 and a "
                    "known dtype required");
    const int64_t n = rows < chunk_rows ? rows : chunk_rows;
    *bytes = (size_t)n * d_ff * (dtype == LSH_BF16 ? 2 : 4);
    return LSH_OK;
}

int check_dmodel(const char* fn, int32_t d_model) {
    if (d_model < 8 || d_model % 8 != 0)
        return fail(LSH_ERR_ARG, "%s: d_model must be a positive multiple of 8 (got %d)", fn,
                    (int)d_model);
    return LSH_OK;
}

}  // namespace

extern "C" {

const char* lsh_last_error(void) { return g_err; }

int lsh_debug_fail_launch(int32_t n) {
    g_err[0] = 0;
    if (n < 0) return fail(LSH_ERR_ARG, "lsh_debug_fail_launch: n must be >= 0 (got %d)", n);
    g_fail_in = n;
    g_injected = false;
    return LSH_OK;
}

size_t lsh_workspace_size(const char* stage, const lsh_shape_t* shape) {
    g_err[0] = 0;
    if (!stage) return fail(LSH_ERR_ARG, "lsh_workspace_size: stage must not be NULL"), 0;
    if (validate(shape)) return 0;
    const Dims d = make_dims(*shape);
    if (!strcmp(stage, "hash")) return hash_workspace_bytes(d);
    if (!strcmp(stage, "sort")) return sort_workspace_bytes(d);
    if (!strcmp(stage, "fwd")) return fwd_layout(d).total;
    if (!strcmp(stage, "fwd_qk")) return fwd_layout(d, true).total;
    if (!strcmp(stage, "fwd_x")) return 2 * projected_bytes(d) + fwd_layout(d).total;
    if (!strcmp(stage, "state")) return state_layout(d).total;
    if (!strcmp(stage, "bwd")) return bwd_layout(d).total;
    fail(LSH_ERR_ARG, "unknown stage '%s' (hash, sort, fwd, fwd_qk, fwd_x, state or bwd)",
         stage);
    return 0;
}

int lsh_hash(const void* qk, const float* R, const lsh_shape_t* shape, int32_t* buckets,
             void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    int rc = validate(shape);
    if (rc) return rc;
    if (empty(shape)) return LSH_OK;
    if (!qk || !R || !buckets) return fail(LSH_ERR_ARG, "lsh_hash: NULL tensor pointer");
    if (misaligned({qk, R, buckets}))
        return fail(LSH_ERR_ARG, "lsh_hash: tensor pointers must be 16-byte aligned");
    const Dims d = make_dims(*shape);
    if ((rc = check_ws("lsh_hash", d, ws, ws_bytes, hash_workspace_bytes(d)))) return rc;
    hipError_t e = launch_hash(qk, R, d, buckets, carve_hash_workspace(ws, d), (hipStream_t)stream,
                               nullptr, nullptr, nullptr);
    if (e == hipSuccess) e = hipGetLastError();
    return e == hipSuccess ? LSH_OK : hip_fail(e, "lsh_hash");
}

int lsh_sort(const int32_t* buckets, const lsh_shape_t* shape, int32_t* perm, int32_t* inv,
             void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    int rc = validate(shape);
    if (rc) return rc;
    if (empty(shape)) return LSH_OK;
    if (!buckets || !perm || !inv) return fail(LSH_ERR_ARG, "lsh_sort: NULL tensor pointer");
    if (misaligned({buckets, perm, inv}))
        return fail(LSH_ERR_ARG, "lsh_sort: tensor pointers must be 16-byte aligned");
    const Dims d = make_dims(*shape);
    if ((rc = check_ws("lsh_sort", d, ws, ws_bytes, sort_workspace_bytes(d)))) return rc;
    hipError_t e = launch_sort(buckets, d, perm, inv, ws, (hipStream_t)stream, nullptr, nullptr,
                               nullptr);
    if (e == hipSuccess) e = hipGetLastError();
    return e == hipSuccess ? LSH_OK : hip_fail(e, "lsh_sort");
}

int lsh_sort_noalloc(const int32_t* buckets, const lsh_shape_t* shape, int32_t* perm, int32_t* inv,
                     void* stream) {
    g_err[0] = 0;
    int rc = validate(shape);
    if (rc) return rc;
    if (empty(shape)) return LSH_OK;
    if (!buckets || !perm || !inv)
        return fail(LSH_ERR_ARG, "lsh_sort_noalloc: NULL tensor pointer");
    if (misaligned({buckets, perm, inv}))
        return fail(LSH_ERR_ARG, "lsh_sort_noalloc: tensor pointers must be 16-byte aligned");
    const Dims d = make_dims(*shape);
    const size_t need = sort_workspace_bytes(d);
    if (need > kSortScratchBytes)
        return fail(LSH_ERR_WORKSPACE,
                    "lsh_sort_noalloc: the shape needs %zu bytes of scratch, the static scratch "
                    "holds %zu (use lsh_sort with a workspace)",
                    need, kSortScratchBytes);
    hipStream_t st = (hipStream_t)stream;
    if (st) {
        int cur = 0, sdev = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess) e = hipStreamGetDevice(st, &sdev);
        if (e != hipSuccess) return hip_fail(e, "lsh_sort_noalloc: device of the stream");
        if (sdev != cur)
            return fail(LSH_ERR_ARG, "lsh_sort_noalloc: the stream belongs to device %d, the "
                                     "current device is %d", sdev, cur);
    }
    void* ws = nullptr;
    hipError_t e = sort_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "lsh_sort_noalloc: scratch address");
    e = launch_sort(buckets, d, perm, inv, ws, st, nullptr, nullptr, nullptr);
    if (e == hipSuccess) e = hipGetLastError();
    return e == hipSuccess ? LSH_OK : hip_fail(e, "lsh_sort_noalloc");
}

int lsh_chunk_attend(const void* qk, const void* v, const int32_t* buckets, const int32_t* perm,
                     const lsh_shape_t* shape, float* o_sorted, float* lse_sorted, void* stream) {
    g_err[0] = 0;
    int rc = validate(shape);
    if (rc) return rc;
    if (empty(shape)) return LSH_OK;
    if (!qk || !v || !buckets || !perm || !o_sorted || !lse_sorted)
        return fail(LSH_ERR_ARG, "lsh_chunk_attend: NULL tensor pointer");
    if (misaligned({qk, v, buckets, perm, o_sorted, lse_sorted}))
        return fail(LSH_ERR_ARG, "lsh_chunk_attend: tensor pointers must be 16-byte aligned");
    const Dims d = make_dims(*shape);
    const OSorted o{o_sorted, false, nullptr};
    hipError_t e = launch_attend(qk, v, buckets, perm, d, o, lse_sorted, (hipStream_t)stream,
                                 nullptr, nullptr, nullptr);
    if (e == hipSuccess) e = hipGetLastError();
    return e == hipSuccess ? LSH_OK : hip_fail(e, "lsh_chunk_attend");
}

int lsh_chunk_attend_qk(const void* q, const void* k, const void* v, const int32_t* buckets_q,
                        const int32_t* buckets_k, const int32_t* perm_q, const int32_t* perm_k,
                        const lsh_shape_t* shape, float* o_sorted, float* lse_sorted,
                        void* stream) {
    g_err[0] = 0;
    int rc = validate(shape);
    if (rc) return rc;
    if (shape->flags & LSH_KEY_NORM)
        return fail(LSH_ERR_ARG, "lsh_chunk_attend_qk: LSH_KEY_NORM belongs to shared queries "
                                 "and keys");
    if (empty(shape)) return LSH_OK;
    if (!q || !k || !v || !buckets_q || !buckets_k || !perm_q || !perm_k || !o_sorted ||
        !lse_sorted)
        return fail(LSH_ERR_ARG, "lsh_chunk_attend_qk: NULL tensor pointer");
    if (misaligned({q, k, v, buckets_q, buckets_k, perm_q, perm_k, o_sorted, lse_sorted}))
        return fail(LSH_ERR_ARG, "lsh_chunk_attend_qk: tensor pointers must be 16-byte aligned");
    const Dims d = make_dims(*shape);
    const OSorted o{o_sorted, false, nullptr};
    const SepQK sep{q, buckets_q, perm_q};
    hipError_t e = launch_attend(k, v, buckets_k, perm_k, d, o, lse_sorted, (hipStream_t)stream,
                                 nullptr, nullptr, nullptr, false, nullptr, &sep);
    if (e == hipSuccess) e = hipGetLastError();
    return e == hipSuccess ? LSH_OK : hip_fail(e, "lsh_chunk_attend_qk");
}

int lsh_unsort_combine(const float* o_sorted, const float* lse_sorted, const int32_t* inv,
                       const lsh_shape_t* shape, void* out, void* stream) {
    g_err[0] = 0;
    int rc = validate(shape);
    if (rc) return rc;
    if (empty(shape)) return LSH_OK;
    if (!o_sorted || !lse_sorted || !inv || !out)
        return fail(LSH_ERR_ARG, "lsh_unsort_combine: NULL tensor pointer");
    if (misaligned({o_sorted, lse_sorted, inv, out}))
        return fail(LSH_ERR_ARG, "lsh_unsort_combine: tensor pointers must be 16-byte aligned");
    const Dims d = make_dims(*shape);
    const OSorted o{(void*)o_sorted, false, nullptr};
    hipError_t e = launch_combine(o, lse_sorted, inv, d, out, (hipStream_t)stream, nullptr,
                                  nullptr, nullptr);
    if (e == hipSuccess) e = hipGetLastError();
    return e == hipSuccess ? LSH_OK : hip_fail(e, "lsh_unsort_combine");
}

int lsh_attention_fwd(const void* qk, const void* v, const float* R, const lsh_shape_t* shape,
                      void* out, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    int rc = validate(shape);
    if (rc) return rc;
    if (empty(shape)) return LSH_OK;
    if (!qk || !v || !R || !out) return fail(LSH_ERR_ARG, "lsh_attention_fwd: NULL tensor pointer");
    if (misaligned({qk, v, R, out}))
        return fail(LSH_ERR_ARG, "lsh_attention_fwd: tensor pointers must be 16-byte aligned");
    return run_fwd(qk, v, R, shape, out, ws, ws_bytes, (hipStream_t)stream, nullptr, nullptr,
                   nullptr);
}

int lsh_attention_fwd_qk(const void* q, const void* k, const void* v, const float* R,
                         const lsh_shape_t* shape, void* out, void* ws, size_t ws_bytes,
                         void* stream) {
    g_err[0] = 0;
    int rc = validate(shape);
    if (rc) return rc;
    if (shape->flags & LSH_KEY_NORM)
        return fail(LSH_ERR_ARG, "lsh_attention_fwd_qk: LSH_KEY_NORM belongs to shared queries "
                                 "and keys");
    if (empty(shape)) return LSH_OK;
    if (!q || !k || !v || !R || !out)
        return fail(LSH_ERR_ARG, "lsh_attention_fwd_qk: NULL tensor pointer");
    if (misaligned({q, k, v, R, out}))
        return fail(LSH_ERR_ARG, "lsh_attention_fwd_qk: tensor pointers must be 16-byte aligned");
    return run_fwd_qk(q, k, v, R, shape, out, ws, ws_bytes, (hipStream_t)stream);
}

int lsh_qkv_project(const void* x, const void* w_qk, const void* w_v, const lsh_shape_t* shape,
                    int32_t d_model, void* qk, void* v, void* stream) {
    g_err[0] = 0;
    int rc = validate(shape);
    if (rc) return rc;
    if ((rc = check_dmodel("lsh_qkv_project", d_model))) return rc;
    if (empty(shape)) return LSH_OK;
    if (!x || !w_qk || !w_v || !qk || !v)
        return fail(LSH_ERR_ARG, "lsh_qkv_project: NULL tensor pointer");
    if (misaligned({x, w_qk, w_v, qk, v}))
        return fail(LSH_ERR_ARG, "lsh_qkv_project: tensor pointers must be 16-byte aligned");
    const Dims d = make_dims(*shape);
    hipError_t e = launch_project(x, w_qk, w_v, d, d_model, qk, v, (hipStream_t)stream);
    return e == hipSuccess ? LSH_OK : hip_fail(e, "lsh_qkv_project");
}

size_t lsh_ffn_workspace_size(int64_t rows, int32_t d_ff, int32_t chunk_rows, int32_t dtype) {
    g_err[0] = 0;
    size_t bytes = 0;
    return ffn_workspace(rows, d_ff, chunk_rows, dtype, &bytes) ? 0 : bytes;
}

int lsh_ffn_chunked(const void* x, const void* w1, const void* b1, const void* w2,
                    const void* b2, int64_t rows, int32_t d_model, int32_t d_ff,
                    int32_t chunk_rows, int32_t dtype, void* out, void* ws, size_t ws_bytes,
                    void* stream) {
    g_err[0] = 0;
    if (d_model < 8 || d_model % 8 != 0)
        return fail(LSH_ERR_ARG, "lsh_ffn_chunked: d_model must be a positive multiple of 8 "
                                 "(got %d)", (int)d_model);
    size_t need = 0;
    int rc = ffn_workspace(rows, d_ff, chunk_rows, dtype, &need);
    if (rc) return rc;
    if (rows == 0) return LSH_OK;
    if (!x || !w1 || !w2 || !out)
        return fail(LSH_ERR_ARG, "lsh_ffn_chunked: NULL tensor pointer");
    if (misaligned({x, w1, w2, out}))
        return fail(LSH_ERR_ARG, "lsh_ffn_chunked: tensor pointers must be 16-byte aligned");
    if (!ws) return fail(LSH_ERR_WORKSPACE, "lsh_ffn_chunked: workspace is NULL");
    if (misaligned({ws})) return fail(LSH_ERR_ARG, "lsh_ffn_chunked: workspace must be 16-byte aligned");
    if (ws_bytes < need)
        return fail(LSH_ERR_WORKSPACE, "lsh_ffn_chunked: workspace has %zu bytes, needs %zu",
                    ws_bytes, need);
    hipError_t e = launch_ffn(x, w1, b1, w2, b2, rows, d_model, d_ff, chunk_rows,
                              dtype == LSH_BF16, out, ws, (hipStream_t)stream);
    return e == hipSuccess ? LSH_OK : hip_fail(e, "lsh_ffn_chunked");
}

int lsh_attention_fwd_x(const void* x, const void* w_qk, const void* w_v, const float* R,
                        const lsh_shape_t* shape, int32_t d_model, void* out, void* ws,
                        size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    int rc = validate(shape);
    if (rc) return rc;
    if ((rc = check_dmodel("lsh_attention_fwd_x", d_model))) return rc;
    if (empty(shape)) return LSH_OK;
    if (!x || !w_qk || !w_v || !R || !out)
        return fail(LSH_ERR_ARG, "lsh_attention_fwd_x: NULL tensor pointer");
    if (misaligned({x, w_qk, w_v, R, out}))
        return fail(LSH_ERR_ARG, "lsh_attention_fwd_x: tensor pointers must be 16-byte aligned");
    const Dims d = make_dims(*shape);
    const size_t pb = projected_bytes(d);
    if ((rc = check_ws("lsh_attention_fwd_x", d, ws, ws_bytes, 2 * pb + fwd_layout(d).total)))
        return rc;
    // the forward's own workspace comes first, so its re-decided count stays
    // the first int32 of ws; the projected tensors follow it
    const size_t fb = fwd_layout(d).total;
    char* qk = (char*)ws + fb;
    char* v = qk + pb;
    hipError_t e = launch_project(x, w_qk, w_v, d, d_model, qk, v, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "lsh_attention_fwd_x: projection");
    return run_fwd(qk, v, R, shape, out, ws, fb, (hipStream_t)stream, nullptr, nullptr, nullptr);
}

int lsh_attention_fwd_train(const void* qk, const void* v, const float* R,
                            const lsh_shape_t* shape, void* out, void* state,
                            size_t state_bytes, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    int rc = validate(shape);
    if (rc) return rc;
    if (empty(shape)) return LSH_OK;
    if (!qk || !v || !R || !out)
        return fail(LSH_ERR_ARG, "lsh_attention_fwd_train: NULL tensor pointer");
    if (misaligned({qk, v, R, out}))
        return fail(LSH_ERR_ARG, "lsh_attention_fwd_train: tensor pointers must be 16-byte aligned");
    const Dims d = make_dims(*shape);
    if ((rc = check_ws("lsh_attention_fwd_train (state)", d, state, state_bytes,
                       state_layout(d).total)))
        return rc;
    return run_fwd(qk, v, R, shape, out, ws, ws_bytes, (hipStream_t)stream, nullptr, nullptr,
                   nullptr, state);
}

int lsh_attention_bwd(const void* qk, const void* v, const void* out, const void* dout,
                      const void* state, size_t state_bytes, const lsh_shape_t* shape, void* dqk,
                      void* dv, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    int rc = validate(shape);
    if (rc) return rc;
    if (empty(shape)) return LSH_OK;
    if (!qk || !v || !out || !dout || !dqk || !dv)
        return fail(LSH_ERR_ARG, "lsh_attention_bwd: NULL tensor pointer");
    if (misaligned({qk, v, out, dout, dqk, dv}))
        return fail(LSH_ERR_ARG, "lsh_attention_bwd: tensor pointers must be 16-byte aligned");
    const Dims d = make_dims(*shape);
    const StateLayout sl = state_layout(d);
    if ((rc = check_ws("lsh_attention_bwd (state)", d, (void*)state, state_bytes, sl.total)))
        return rc;
    const BwdLayout bl = bwd_layout(d);
    if ((rc = check_ws("lsh_attention_bwd", d, ws, ws_bytes, bl.total))) return rc;
    const char* sb = (const char*)state;
    char* wb = (char*)ws;
    float* rn = d.key_norm ? (float*)(wb + bl.rn) : nullptr;
    BwdArgs a{qk, v, out, dout,
              (const int32_t*)(sb + sl.perm), (const int32_t*)(sb + sl.buckets),
              (const float*)(sb + sl.z), (float*)(wb + bl.dvec), rn, (float*)(wb + bl.dx),
              (float*)(wb + bl.dv), dqk, dv};
    hipError_t e = hipSuccess;
    if (rn) e = launch_key_rnorm(qk, d, rn, (hipStream_t)stream);
    if (e == hipSuccess) e = launch_backward(a, d, fused_packed(d), (hipStream_t)stream);
    return e == hipSuccess ? LSH_OK : hip_fail(e, "lsh_attention_bwd");
}

int lsh_attention_fwd_timed(const void* qk, const void* v, const float* R,
                            const lsh_shape_t* shape, void* out, void* ws, size_t ws_bytes,
                            void* stream, float* kernel_ms, const char** kernel_names,
                            int32_t max_kernels, int32_t* n_kernels) {
    g_err[0] = 0;
    int rc = validate(shape);
    if (rc) return rc;
    if (!kernel_ms || !n_kernels || max_kernels < 1)
        return fail(LSH_ERR_ARG, "lsh_attention_fwd_timed: NULL timing output");
    *n_kernels = 0;
    if (empty(shape)) return LSH_OK;
    if (!qk || !v || !R || !out)
        return fail(LSH_ERR_ARG, "lsh_attention_fwd_timed: NULL tensor pointer");
    if (misaligned({qk, v, R, out}))
        return fail(LSH_ERR_ARG, "lsh_attention_fwd_timed: tensor pointers must be 16-byte aligned");
    constexpr int kMaxMarks = 16;
    hipEvent_t ev[kMaxMarks + 1];
    int created = 0;
    hipError_t e = hipSuccess;
    for (; created < kMaxMarks + 1; ++created)
        if ((e = hipEventCreate(&ev[created])) != hipSuccess) break;
    hipStream_t st = (hipStream_t)stream;
    const char* names[kMaxMarks] = {};
    int nev = 0;
    if (e == hipSuccess) e = hipEventRecord(ev[0], st);
    if (e == hipSuccess) {
        rc = run_fwd(qk, v, R, shape, out, ws, ws_bytes, st, ev, &nev, names);
        if (rc == LSH_OK) {
            e = hipEventSynchronize(ev[nev]);
            for (int k = 0; e == hipSuccess && k < nev && k < max_kernels; ++k) {
                e = hipEventElapsedTime(&kernel_ms[k], ev[k], ev[k + 1]);
                if (kernel_names) kernel_names[k] = names[k];
            }
            *n_kernels = nev < max_kernels ? nev : max_kernels;
        }
    }
    for (int k = 0; k < created; ++k) (void)hipEventDestroy(ev[k]);
    if (rc) return rc;
    return e == hipSuccess ? LSH_OK : hip_fail(e, "lsh_attention_fwd_timed");
}

}  // extern "C"
