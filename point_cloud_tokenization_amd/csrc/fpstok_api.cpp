// C ABI of libfpstok (declared and documented in include/fpstok.h): argument
// validation, workspace carve-up and kernel launches.  Validation happens on
// the host before any HIP call, so an invalid call never touches the device.
#include "fpstok.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "fpstok_internal.h"

#define FPSTOK_API extern "C" __attribute__((visibility("default")))

namespace fpstok {

static thread_local char g_last_error[512] = "";

static fpstok_status fail(fpstok_status st, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));

static fpstok_status fail(fpstok_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

static fpstok_status ok() {
    g_last_error[0] = '\0';
    return FPSTOK_OK;
}

static fpstok_status hip_fail(hipError_t e, const char* what) {
    return fail(FPSTOK_EHIP, "%s: %s", what, hipGetErrorString(e));
}

static_assert(kKnnMaxK == FPSTOK_MAX_K, "kNN list bound");
static_assert(kNoAllocBytes == FPSTOK_NOALLOC_MAX_WORKSPACE, "scratch region size");

// Polls before a wait between workgroups gives up (fpstok_debug_set_spin_limit).
static std::atomic<uint32_t> g_spin_limit{kDefaultSpinLimit};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WorkspaceLayout workspace_layout(int64_t B, int64_t N, int P, int C, int coords_dtype,
                                 int features_dtype) {
    WorkspaceLayout L{};
    if (B <= 0) return L;
    const int64_t nn = N > 0 ? N : 0;
    L.max_chunks = (nn + kChunk - 1) / kChunk + B;
    size_t at = 0;
    L.header = at;
    at += align256(64 * sizeof(int32_t));
    L.chunk_ev = at;
    at += align256((size_t)L.max_chunks * sizeof(int32_t));
    L.chunk_beg = at;
    at += align256((size_t)L.max_chunks * sizeof(int32_t));
    L.max_pool_chunks = nn / kPoolChunk + B;
    L.pool_ev = at;
    at += align256((size_t)L.max_pool_chunks * sizeof(int32_t));
    L.pool_beg = at;
    at += align256((size_t)L.max_pool_chunks * sizeof(int32_t));
    L.chunk_part = at;
    at += align256((size_t)L.max_pool_chunks * sizeof(int32_t));
    L.big_ev = at;
    at += align256(2 * (size_t)B * sizeof(int32_t));
    L.mind = at;
    at += align256((size_t)nn * sizeof(float));
    L.near = at;
    at += align256((size_t)nn * sizeof(int32_t));
    L.perm = at;
    at += align256((size_t)nn * sizeof(int32_t));
    L.max_items = sample_max_items(B, nn);
    L.item_ev = at;
    at += align256((size_t)L.max_items * sizeof(int32_t));
    L.item_g = at;
    at += align256((size_t)L.max_items * sizeof(int32_t));
    L.gang_rec = at;
    at += align256((size_t)L.max_items * 2 * kGangRecWords * sizeof(unsigned long long));
    L.shard_cells = at;
    at += align256((size_t)L.max_items * (size_t)(P + 1) * sizeof(int32_t));
    L.max_parts = nn / kGangPulsesPerShard + 1;
    L.part = at;
    at += align256((size_t)L.max_parts * (size_t)P * (size_t)(C + 2) * sizeof(double));
    L.coords32 = at;
    if (coords_dtype != FPSTOK_F32) at += align256((size_t)nn * 4 * sizeof(float));
    L.feat32 = at;
    if (features_dtype != FPSTOK_F32) at += align256((size_t)nn * (size_t)C * sizeof(float));
    L.total = at;
    return L;
}

// Checks shared by every compute call.  `need_features`: the call reads the
// feature matrix (0: no, 1: yes).
static fpstok_status check_common(const fpstok_batch* bt, const fpstok_params* pr,
                                  bool need_features, bool need_weights_col) {
    if (!bt) return fail(FPSTOK_EINVAL, "batch is NULL");
    if (!pr) return fail(FPSTOK_EINVAL, "params is NULL");
    if (bt->num_events < 0) return fail(FPSTOK_EINVAL, "num_events < 0");
    if (bt->num_points < 0) return fail(FPSTOK_EINVAL, "num_points < 0");
    if (bt->num_points >= ((int64_t)1 << 31))
        return fail(FPSTOK_EUNSUPPORTED, "num_points >= 2^31 (indices are int32)");
    if (bt->num_events >= ((int64_t)1 << 31))
        return fail(FPSTOK_EUNSUPPORTED, "num_events >= 2^31");
    if (pr->num_patches < 1 || pr->num_patches > FPSTOK_MAX_PATCHES)
        return fail(FPSTOK_EINVAL, "num_patches must be in [1, %d]", FPSTOK_MAX_PATCHES);
    if (pr->assign_mode != FPSTOK_VORONOI && pr->assign_mode != FPSTOK_KNN)
        return fail(FPSTOK_EINVAL, "unknown assign_mode %d", pr->assign_mode);
    if (pr->assign_mode == FPSTOK_KNN && (pr->k < 1 || pr->k > FPSTOK_MAX_K))
        return fail(FPSTOK_EINVAL, "k must be in [1, %d] in kNN mode", FPSTOK_MAX_K);
    if (pr->lloyd_iters < 0 || pr->lloyd_iters > FPSTOK_MAX_LLOYD)
        return fail(FPSTOK_EINVAL, "lloyd_iters must be in [0, %d]", FPSTOK_MAX_LLOYD);
    if (pr->pool_weighted != 0 && pr->pool_weighted != 1)
        return fail(FPSTOK_EINVAL, "pool_weighted must be 0 or 1");
    if (bt->coords_dtype < FPSTOK_F32 || bt->coords_dtype > FPSTOK_BF16)
        return fail(FPSTOK_EINVAL, "coords_dtype must be FPSTOK_F32, FPSTOK_F16 or FPSTOK_BF16");
    if (bt->features_dtype < FPSTOK_F32 || bt->features_dtype > FPSTOK_BF16)
        return fail(FPSTOK_EINVAL, "features_dtype must be FPSTOK_F32, FPSTOK_F16 or FPSTOK_BF16");
    if (bt->num_events == 0) return FPSTOK_OK;
    if (!bt->offsets) return fail(FPSTOK_EINVAL, "offsets is NULL");
    if (bt->num_points > 0) {
        if (!bt->coords) return fail(FPSTOK_EINVAL, "coords is NULL");
        const uintptr_t ca = bt->coords_dtype == FPSTOK_F32 ? 15u : 7u;
        if (((uintptr_t)bt->coords & ca) != 0)
            return fail(FPSTOK_EINVAL, "coords must be %d-byte aligned", (int)ca + 1);
    }
    if (need_features) {
        if (bt->num_features < 1) return fail(FPSTOK_EINVAL, "num_features must be >= 1");
        if (bt->num_points > 0 && !bt->features) return fail(FPSTOK_EINVAL, "features is NULL");
        const uintptr_t fa = bt->features_dtype == FPSTOK_F32 ? 3u : 1u;
        if (bt->features && ((uintptr_t)bt->features & fa) != 0)
            return fail(FPSTOK_EINVAL, "features must be %d-byte aligned", (int)fa + 1);
    }
    if (need_features || need_weights_col) {
        if (bt->charge_col < -1 || (bt->num_features >= 1 && bt->charge_col >= bt->num_features))
            return fail(FPSTOK_EINVAL, "charge_col must be -1 or in [0, num_features)");
        if (bt->charge_col >= 0 && bt->num_features < 1)
            return fail(FPSTOK_EINVAL, "charge_col set but num_features < 1");
        if (bt->charge_col >= 0 && bt->num_points > 0 && !bt->features)
            return fail(FPSTOK_EINVAL, "charge_col set but features is NULL");
    }
    return FPSTOK_OK;
}

static WorkspaceLayout batch_layout(const fpstok_batch* bt, int P) {
    return workspace_layout(bt->num_events, bt->num_points, P,
                            bt->num_features > 0 ? bt->num_features : 1, bt->coords_dtype,
                            bt->features_dtype);
}

static fpstok_status check_ws(const fpstok_batch* bt, const fpstok_params* pr, void* ws,
                              size_t ws_bytes, WorkspaceLayout& L) {
    L = batch_layout(bt, pr->num_patches);
    if (L.total == 0) return FPSTOK_OK;
    if (!ws) return fail(FPSTOK_EWORKSPACE, "workspace is NULL (need %zu bytes)", L.total);
    if (ws_bytes < L.total)
        return fail(FPSTOK_EWORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, L.total);
    if (((uintptr_t)ws & 255u) != 0)
        return fail(FPSTOK_EINVAL, "workspace must be 256-byte aligned");
    return FPSTOK_OK;
}

template <class T>
static T* at(void* ws, size_t off) {
    return (T*)((char*)ws + off);
}

// 16-bit inputs the call reads (coordinates, features) are upcast into
// their float32 copies in the workspace, and `bt` is pointed at a copy of
// the batch that names those instead (everything else unchanged).
static fpstok_status stage_inputs(const fpstok_batch*& bt, fpstok_batch& tmp, bool coords,
                                  bool features, void* ws, const WorkspaceLayout& L,
                                  hipStream_t s) {
    const int64_t N = bt->num_points;
    const bool c16 = coords && bt->coords_dtype != FPSTOK_F32 && N > 0;
    const bool f16 = features && bt->features_dtype != FPSTOK_F32 && N > 0 && bt->features;
    if (!c16 && !f16) return FPSTOK_OK;
    tmp = *bt;
    float* c32 = at<float>(ws, L.coords32);
    float* f32 = at<float>(ws, L.feat32);
    const hipError_t e =
        launch_upcast(c16 ? bt->coords : nullptr, c16 ? N * 4 : 0, bt->coords_dtype, c32,
                      f16 ? bt->features : nullptr, f16 ? N * (int64_t)bt->num_features : 0,
                      bt->features_dtype, f32, s);
    if (e != hipSuccess) return hip_fail(e, "upcast kernel launch");
    if (c16) {
        tmp.coords = c32;
        tmp.coords_dtype = FPSTOK_F32;
    }
    if (f16) {
        tmp.features = f32;
        tmp.features_dtype = FPSTOK_F32;
    }
    bt = &tmp;
    return FPSTOK_OK;
}

static SampleArgs sample_args(const fpstok_batch* bt, const fpstok_params* pr,
                              const int32_t* start_idx, int32_t* centroid_idx, float* centroids,
                              int32_t* token_count, int32_t* assign, void* ws,
                              const WorkspaceLayout& L) {
    SampleArgs a{};
    a.coords = (const float4*)bt->coords;
    a.offsets = bt->offsets;
    a.N = bt->num_points;
    a.B = bt->num_events;
    a.P = pr->num_patches;
    a.start_idx = start_idx;
    a.centroid_idx = centroid_idx;
    a.centroids = (float4*)centroids;
    a.token_count = token_count;
    a.assign = assign;
    a.ws_mind = at<float>(ws, L.mind);
    a.ws_near = at<int32_t>(ws, L.near);
    a.direct = bt->max_event_points > 0 && bt->max_event_points <= kFpsCapPulses ? 1 : 0;
    a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    a.header = at<int32_t>(ws, L.header);
    a.item_ev = at<int32_t>(ws, L.item_ev);
    a.item_g = at<int32_t>(ws, L.item_g);
    a.gang_rec = at<unsigned long long>(ws, L.gang_rec);
    a.shard_cells = at<int32_t>(ws, L.shard_cells);
    a.gang_part = at<double>(ws, L.part);
    return a;
}

static PoolArgs pool_args(const fpstok_batch* bt, const fpstok_params* pr,
                          const int32_t* token_count, const int32_t* assign,
                          const int32_t* knn_idx, float* pooled, int32_t* cell_count, void* ws,
                          const WorkspaceLayout& L) {
    PoolArgs a{};
    a.features = (const float*)bt->features;
    a.offsets = bt->offsets;
    a.N = bt->num_points;
    a.C = bt->num_features;
    a.weight_col = pr->pool_weighted ? bt->charge_col : -1;
    a.P = pr->num_patches;
    a.k = pr->k;
    a.token_count = token_count;
    a.assign = assign;
    a.knn_idx = knn_idx;
    a.pooled = pooled;
    a.cell_count = cell_count;
    a.perm = at<int32_t>(ws, L.perm);
    a.header = at<int32_t>(ws, L.header);
    a.chunk_ev = at<int32_t>(ws, L.pool_ev);
    a.chunk_beg = at<int32_t>(ws, L.pool_beg);
    a.chunk_part = at<int32_t>(ws, L.chunk_part);
    a.big_ev = at<int32_t>(ws, L.big_ev);
    a.B = bt->num_events;
    // events of more than one chunk are finished by the combine kernel, whose
    // blocks hold one thread per (field, slot); when the caller's bound on
    // event size rules them out the combine kernel is not launched, and an
    // event that breaks the bound is summed whole by its first chunk's
    // workgroup (slower, still correct)
    const bool no_big = bt->max_event_points > 0 && bt->max_event_points <= kPoolChunk;
    a.whole = no_big || bt->num_features + 2 > 256 ? 1 : 0;
    a.part = at<double>(ws, L.part);
    return a;
}

// The Lloyd rounds once the assign chunk list is planned.
static hipError_t run_lloyd(const fpstok_batch* bt, const fpstok_params* pr, float* centroids,
                            const int32_t* token_count, int32_t* assign, void* ws,
                            const WorkspaceLayout& L, hipStream_t s) {
    LloydArgs u{};
    u.coords = (const float4*)bt->coords;
    u.features = (const float*)bt->features;
    u.offsets = bt->offsets;
    u.N = bt->num_points;
    u.C = bt->num_features;
    u.charge_col = bt->charge_col;
    u.P = pr->num_patches;
    u.centroids = (float4*)centroids;
    u.token_count = token_count;
    u.assign = assign;
    u.perm = at<int32_t>(ws, L.perm);
    AssignArgs a{};
    a.coords = u.coords;
    a.offsets = bt->offsets;
    a.N = bt->num_points;
    a.P = pr->num_patches;
    a.centroids = (const float4*)centroids;
    a.token_count = token_count;
    a.assign = assign;
    a.header = at<int32_t>(ws, L.header);
    a.chunk_ev = at<int32_t>(ws, L.chunk_ev);
    a.chunk_beg = at<int32_t>(ws, L.chunk_beg);
    a.skip_small = 1;
    for (int it = 0; it < pr->lloyd_iters; ++it) {
        hipError_t e = launch_lloyd_update(u, bt->num_events, s);
        if (e != hipSuccess) return e;
        e = launch_assign(a, L.max_chunks, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// The pooling kernels once the pooling chunk list is planned.
static hipError_t run_pool(const fpstok_batch* bt, const fpstok_params* pr, const PoolArgs& a,
                           const WorkspaceLayout& L, hipStream_t s) {
    if (pr->assign_mode != FPSTOK_VORONOI) return launch_pool_knn(a, bt->num_events, s);
    hipError_t e = launch_pool_voronoi(a, L.max_pool_chunks, s);
    if (e == hipSuccess) e = launch_pool_combine(a, s);
    return e;
}

}  // namespace fpstok

using namespace fpstok;

FPSTOK_API size_t fpstok_workspace_size(const fpstok_batch* batch, const fpstok_params* params) {
    if (!batch) return 0;
    int P = params ? params->num_patches : FPSTOK_MAX_PATCHES;
    if (P < 1 || P > FPSTOK_MAX_PATCHES) P = FPSTOK_MAX_PATCHES;
    return batch_layout(batch, P).total;
}

FPSTOK_API fpstok_status fpstok_sample(const fpstok_batch* bt, const fpstok_params* pr,
                                       const int32_t* start_idx, int32_t* centroid_idx,
                                       float* centroids, int32_t* token_count, int32_t* assign,
                                       void* ws, size_t ws_bytes, void* stream) {
    fpstok_status st = check_common(bt, pr, false, false);
    if (st != FPSTOK_OK) return st;
    if (bt->num_events == 0) return ok();
    if (!centroid_idx || !centroids || !token_count)
        return fail(FPSTOK_EINVAL, "centroid_idx, centroids and token_count are required");
    if (((uintptr_t)centroids & 15u) != 0)
        return fail(FPSTOK_EINVAL, "centroids must be 16-byte aligned");
    WorkspaceLayout L;
    if ((st = check_ws(bt, pr, ws, ws_bytes, L)) != FPSTOK_OK) return st;
    fpstok_batch staged;
    if ((st = stage_inputs(bt, staged, true, false, ws, L, (hipStream_t)stream)) != FPSTOK_OK)
        return st;
    const SampleArgs a = sample_args(bt, pr, start_idx, centroid_idx, centroids, token_count,
                                     assign, ws, L);
    hipError_t e = launch_sample(a, bt->num_events, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "sample kernel launch");
    return ok();
}

FPSTOK_API fpstok_status fpstok_assign(const fpstok_batch* bt, const fpstok_params* pr,
                                       const float* centroids, const int32_t* token_count,
                                       int32_t* assign, void* ws, size_t ws_bytes, void* stream) {
    fpstok_status st = check_common(bt, pr, false, false);
    if (st != FPSTOK_OK) return st;
    if (bt->num_events == 0) return ok();
    if (!centroids || !token_count || !assign)
        return fail(FPSTOK_EINVAL, "centroids, token_count and assign are required");
    if (((uintptr_t)centroids & 15u) != 0)
        return fail(FPSTOK_EINVAL, "centroids must be 16-byte aligned");
    WorkspaceLayout L;
    if ((st = check_ws(bt, pr, ws, ws_bytes, L)) != FPSTOK_OK) return st;
    fpstok_batch staged;
    if ((st = stage_inputs(bt, staged, true, false, ws, L, (hipStream_t)stream)) != FPSTOK_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_plan(bt->offsets, bt->num_events, bt->num_points, ws, L, s);
    if (e != hipSuccess) return hip_fail(e, "plan kernel launch");
    AssignArgs a{};
    a.coords = (const float4*)bt->coords;
    a.offsets = bt->offsets;
    a.N = bt->num_points;
    a.P = pr->num_patches;
    a.centroids = (const float4*)centroids;
    a.token_count = token_count;
    a.assign = assign;
    a.header = at<int32_t>(ws, L.header);
    a.chunk_ev = at<int32_t>(ws, L.chunk_ev);
    a.chunk_beg = at<int32_t>(ws, L.chunk_beg);
    a.skip_small = 0;
    e = launch_assign(a, L.max_chunks, s);
    if (e != hipSuccess) return hip_fail(e, "assign kernel launch");
    return ok();
}

FPSTOK_API fpstok_status fpstok_knn(const fpstok_batch* bt, const fpstok_params* pr,
                                    const float* centroids, const int32_t* token_count,
                                    int32_t* knn_idx, void* ws, size_t ws_bytes, void* stream) {
    fpstok_status st = check_common(bt, pr, false, false);
    if (st != FPSTOK_OK) return st;
    if (pr->k < 1 || pr->k > FPSTOK_MAX_K)
        return fail(FPSTOK_EINVAL, "k must be in [1, %d]", FPSTOK_MAX_K);
    if (bt->num_events == 0) return ok();
    if (!centroids || !token_count || !knn_idx)
        return fail(FPSTOK_EINVAL, "centroids, token_count and knn_idx are required");
    if (((uintptr_t)centroids & 15u) != 0)
        return fail(FPSTOK_EINVAL, "centroids must be 16-byte aligned");
    WorkspaceLayout L;
    if ((st = check_ws(bt, pr, ws, ws_bytes, L)) != FPSTOK_OK) return st;
    fpstok_batch staged;
    if ((st = stage_inputs(bt, staged, true, false, ws, L, (hipStream_t)stream)) != FPSTOK_OK)
        return st;
    KnnArgs a{};
    a.coords = (const float4*)bt->coords;
    a.offsets = bt->offsets;
    a.N = bt->num_points;
    a.P = pr->num_patches;
    a.k = pr->k;
    a.centroids = (const float4*)centroids;
    a.token_count = token_count;
    a.knn_idx = knn_idx;
    hipError_t e = launch_knn(a, bt->num_events, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "knn kernel launch");
    return ok();
}

FPSTOK_API fpstok_status fpstok_lloyd(const fpstok_batch* bt, const fpstok_params* pr,
                                      float* centroids, const int32_t* token_count,
                                      int32_t* assign, void* ws, size_t ws_bytes, void* stream) {
    fpstok_status st = check_common(bt, pr, false, true);
    if (st != FPSTOK_OK) return st;
    if (bt->num_events == 0 || pr->lloyd_iters == 0) return ok();
    if (!centroids || !token_count || !assign)
        return fail(FPSTOK_EINVAL, "centroids, token_count and assign are required");
    if (((uintptr_t)centroids & 15u) != 0)
        return fail(FPSTOK_EINVAL, "centroids must be 16-byte aligned");
    WorkspaceLayout L;
    if ((st = check_ws(bt, pr, ws, ws_bytes, L)) != FPSTOK_OK) return st;
    fpstok_batch staged;
    if ((st = stage_inputs(bt, staged, true, bt->charge_col >= 0, ws, L, (hipStream_t)stream)) != FPSTOK_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_plan(bt->offsets, bt->num_events, bt->num_points, ws, L, s);
    if (e != hipSuccess) return hip_fail(e, "plan kernel launch");
    e = run_lloyd(bt, pr, centroids, token_count, assign, ws, L, s);
    if (e != hipSuccess) return hip_fail(e, "lloyd kernel launch");
    return ok();
}

FPSTOK_API fpstok_status fpstok_pool(const fpstok_batch* bt, const fpstok_params* pr,
                                     const int32_t* token_count, const int32_t* assign,
                                     const int32_t* knn_idx, float* pooled, int32_t* cell_count,
                                     void* ws, size_t ws_bytes, void* stream) {
    fpstok_status st = check_common(bt, pr, true, false);
    if (st != FPSTOK_OK) return st;
    if (bt->num_events == 0) return ok();
    if (!token_count || !pooled) return fail(FPSTOK_EINVAL, "token_count and pooled are required");
    if (pr->assign_mode == FPSTOK_VORONOI && !assign && bt->num_points > 0)
        return fail(FPSTOK_EINVAL, "assign is required in Voronoi mode");
    if (pr->assign_mode == FPSTOK_KNN && !knn_idx)
        return fail(FPSTOK_EINVAL, "knn_idx is required in kNN mode");
    WorkspaceLayout L;
    if ((st = check_ws(bt, pr, ws, ws_bytes, L)) != FPSTOK_OK) return st;
    fpstok_batch staged;
    if ((st = stage_inputs(bt, staged, false, true, ws, L, (hipStream_t)stream)) != FPSTOK_OK)
        return st;
    const PoolArgs a = pool_args(bt, pr, token_count, assign, knn_idx, pooled, cell_count, ws, L);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (pr->assign_mode == FPSTOK_VORONOI) {
        e = launch_plan_pool(bt->offsets, bt->num_events, bt->num_points, ws, L, a, s);
        if (e != hipSuccess) return hip_fail(e, "plan kernel launch");
    }
    e = run_pool(bt, pr, a, L, s);
    if (e != hipSuccess) return hip_fail(e, "pool kernel launch");
    return ok();
}

static fpstok_status check_pack(int64_t B, int32_t P, int32_t D) {
    if (B < 0) return fail(FPSTOK_EINVAL, "num_events < 0");
    if (P < 1 || P > FPSTOK_MAX_PATCHES)
        return fail(FPSTOK_EINVAL, "num_patches must be in [1, %d]", FPSTOK_MAX_PATCHES);
    if (D < 1) return fail(FPSTOK_EINVAL, "row_width must be >= 1");
    if (B >= ((int64_t)1 << 31) / P) return fail(FPSTOK_EUNSUPPORTED, "num_events * num_patches >= 2^31");
    if (B * (int64_t)P * D >= ((int64_t)1 << 62)) return fail(FPSTOK_EUNSUPPORTED, "rows too large");
    return FPSTOK_OK;
}

FPSTOK_API fpstok_status fpstok_pack(int64_t num_events, int32_t num_patches, int32_t row_width,
                                     const int32_t* token_count, const float* rows,
                                     float* packed, int32_t* doc_id, int32_t* cu_seqlens,
                                     void* stream) {
    fpstok_status st = check_pack(num_events, num_patches, row_width);
    if (st != FPSTOK_OK) return st;
    if (!cu_seqlens) return fail(FPSTOK_EINVAL, "cu_seqlens is NULL");
    if (num_events > 0 && (!token_count || !rows || !packed))
        return fail(FPSTOK_EINVAL, "token_count, rows and packed are required");
    hipError_t e = launch_pack(num_events, num_patches, row_width, token_count, rows, packed,
                               doc_id, cu_seqlens, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "pack kernel launch");
    return ok();
}

FPSTOK_API fpstok_status fpstok_unpack(int64_t num_events, int32_t num_patches, int32_t row_width,
                                       const int32_t* token_count, const int32_t* cu_seqlens,
                                       const float* packed, float* rows, void* stream) {
    fpstok_status st = check_pack(num_events, num_patches, row_width);
    if (st != FPSTOK_OK) return st;
    if (num_events == 0) return ok();
    if (!token_count || !cu_seqlens || !packed || !rows)
        return fail(FPSTOK_EINVAL, "token_count, cu_seqlens, packed and rows are required");
    hipError_t e = launch_unpack(num_events, num_patches, row_width, token_count, cu_seqlens,
                                 packed, rows, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "unpack kernel launch");
    return ok();
}

FPSTOK_API fpstok_status fpstok_pool_backward(const fpstok_batch* bt, const fpstok_params* pr,
                                              const int32_t* token_count, const int32_t* assign,
                                              const int32_t* knn_idx, const float* pooled,
                                              const float* grad_pooled, float* grad_features,
                                              void* ws, size_t ws_bytes, void* stream) {
    fpstok_status st = check_common(bt, pr, true, false);
    if (st != FPSTOK_OK) return st;
    if (bt->num_events == 0) return ok();
    if (!token_count || !pooled || !grad_pooled)
        return fail(FPSTOK_EINVAL, "token_count, pooled and grad_pooled are required");
    if (bt->num_points > 0 && !grad_features) return fail(FPSTOK_EINVAL, "grad_features is NULL");
    if (pr->assign_mode == FPSTOK_VORONOI && !assign && bt->num_points > 0)
        return fail(FPSTOK_EINVAL, "assign is required in Voronoi mode");
    if (pr->assign_mode == FPSTOK_KNN && !knn_idx)
        return fail(FPSTOK_EINVAL, "knn_idx is required in kNN mode");
    WorkspaceLayout L;
    if ((st = check_ws(bt, pr, ws, ws_bytes, L)) != FPSTOK_OK) return st;
    fpstok_batch staged;
    if ((st = stage_inputs(bt, staged, false, true, ws, L, (hipStream_t)stream)) != FPSTOK_OK)
        return st;
    PoolBwdArgs a{};
    a.features = (const float*)bt->features;
    a.offsets = bt->offsets;
    a.N = bt->num_points;
    a.C = bt->num_features;
    a.wcol = pr->pool_weighted ? bt->charge_col : -1;
    a.P = pr->num_patches;
    a.mode = pr->assign_mode == FPSTOK_KNN ? 1 : 0;
    a.k = pr->assign_mode == FPSTOK_KNN ? pr->k : 1;
    a.token_count = token_count;
    a.assign = assign;
    a.knn_idx = knn_idx;
    a.pooled = pooled;
    a.grad_pooled = grad_pooled;
    a.grad = grad_features;
    a.perm = at<int32_t>(ws, L.perm);
    hipError_t e = launch_pool_backward(a, bt->num_events, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "pool backward kernel launch");
    return ok();
}

FPSTOK_API fpstok_status fpstok_random_start(const int64_t* offsets, int64_t num_events,
                                             uint64_t seed, uint64_t step, int32_t* start_idx,
                                             void* stream) {
    if (num_events < 0) return fail(FPSTOK_EINVAL, "num_events < 0");
    if (num_events == 0) return ok();
    if (!offsets || !start_idx) return fail(FPSTOK_EINVAL, "offsets and start_idx are required");
    if (num_events >= ((int64_t)1 << 31)) return fail(FPSTOK_EUNSUPPORTED, "num_events >= 2^31");
    hipError_t e = launch_random_start(offsets, num_events, seed, step, start_idx,
                                       (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "random start kernel launch");
    return ok();
}

// Argument checks of fpstok_tokenize and fpstok_tokenize_noalloc, the workspace aside.
static fpstok_status check_tokenize(const fpstok_batch* bt, const fpstok_params* pr,
                                    int32_t* centroid_idx, float* centroids,
                                    int32_t* token_count, int32_t* assign, int32_t* knn_idx,
                                    float* pooled) {
    fpstok_status st = check_common(bt, pr, true, true);
    if (st != FPSTOK_OK) return st;
    if (bt->num_events == 0) return FPSTOK_OK;
    if (!centroid_idx || !centroids || !token_count || !pooled)
        return fail(FPSTOK_EINVAL, "centroid_idx, centroids, token_count and pooled are required");
    if (((uintptr_t)centroids & 15u) != 0)
        return fail(FPSTOK_EINVAL, "centroids must be 16-byte aligned");
    const bool voronoi = pr->assign_mode == FPSTOK_VORONOI;
    if ((voronoi || pr->lloyd_iters > 0) && !assign && bt->num_points > 0)
        return fail(FPSTOK_EINVAL, "assign is required in Voronoi mode and for Lloyd");
    if (!voronoi && !knn_idx) return fail(FPSTOK_EINVAL, "knn_idx is required in kNN mode");
    if (!voronoi && (pr->k < 1 || pr->k > FPSTOK_MAX_K))
        return fail(FPSTOK_EINVAL, "k must be in [1, %d]", FPSTOK_MAX_K);
    return FPSTOK_OK;
}

// The tokenizer's launches on a checked workspace.
static fpstok_status run_tokenize(const fpstok_batch* bt, const fpstok_params* pr,
                                  const int32_t* start_idx, int32_t* centroid_idx,
                                  float* centroids, int32_t* token_count, int32_t* assign,
                                  int32_t* knn_idx, float* pooled, int32_t* cell_count, void* ws,
                                  const WorkspaceLayout& L, void* stream) {
    const bool voronoi = pr->assign_mode == FPSTOK_VORONOI;
    const SampleArgs a = sample_args(bt, pr, start_idx, centroid_idx, centroids, token_count,
                                     assign, ws, L);
    hipStream_t s = (hipStream_t)stream;
    if (!voronoi || pr->lloyd_iters > 0) {
        // sample -> Lloyd -> [kNN] -> pool on the same stream and workspace,
        // every work list planned by one launch
        const PoolArgs p = pool_args(bt, pr, token_count, assign, knn_idx, pooled, cell_count, ws,
                                     L);
        hipError_t e = hipSuccess;
        // nothing to plan: no FPS work list (event-size bound), no Lloyd
        // chunks, and kNN pooling needs no chunk list
        if (!a.direct || pr->lloyd_iters > 0 || voronoi) {
            e = launch_plan_all(a, bt->num_events, ws, L, p, pr->lloyd_iters > 0, voronoi, s);
            if (e != hipSuccess) return hip_fail(e, "plan kernel launch");
        }
        e = launch_sample_items(a, bt->num_events, s);
        if (e != hipSuccess) return hip_fail(e, "sample kernel launch");
        e = run_lloyd(bt, pr, centroids, token_count, assign, ws, L, s);
        if (e != hipSuccess) return hip_fail(e, "lloyd kernel launch");
        if (!voronoi) {
            // the lists and their pooling in one launch
            KnnArgs k{};
            k.coords = (const float4*)bt->coords;
            k.offsets = bt->offsets;
            k.N = bt->num_points;
            k.P = pr->num_patches;
            k.k = pr->k;
            k.centroids = (const float4*)centroids;
            k.token_count = token_count;
            k.knn_idx = knn_idx;
            k.features = p.features;
            k.C = p.C;
            k.weight_col = p.weight_col;
            k.pooled = pooled;
            k.cell_count = cell_count;
            e = launch_knn(k, bt->num_events, s);
            if (e != hipSuccess) return hip_fail(e, "knn kernel launch");
            return ok();
        }
        e = run_pool(bt, pr, p, L, s);
        if (e != hipSuccess) return hip_fail(e, "pool kernel launch");
        return ok();
    }
    const PoolArgs p = pool_args(bt, pr, token_count, assign, nullptr, pooled, cell_count, ws, L);
    hipError_t e = launch_tokenize(a, p, bt->num_events, s);
    if (e != hipSuccess) return hip_fail(e, "tokenize kernel launch");
    return ok();
}

FPSTOK_API fpstok_status fpstok_tokenize(const fpstok_batch* bt, const fpstok_params* pr,
                                         const int32_t* start_idx, int32_t* centroid_idx,
                                         float* centroids, int32_t* token_count, int32_t* assign,
                                         int32_t* knn_idx, float* pooled, int32_t* cell_count,
                                         void* ws, size_t ws_bytes, void* stream) {
    fpstok_status st = check_tokenize(bt, pr, centroid_idx, centroids, token_count, assign,
                                      knn_idx, pooled);
    if (st != FPSTOK_OK) return st;
    if (bt->num_events == 0) return ok();
    WorkspaceLayout L;
    if ((st = check_ws(bt, pr, ws, ws_bytes, L)) != FPSTOK_OK) return st;
    fpstok_batch staged;
    if ((st = stage_inputs(bt, staged, true, true, ws, L, (hipStream_t)stream)) != FPSTOK_OK)
        return st;
    return run_tokenize(bt, pr, start_idx, centroid_idx, centroids, token_count, assign, knn_idx,
                        pooled, cell_count, ws, L, stream);
}

FPSTOK_API fpstok_status fpstok_tokenize_noalloc(const fpstok_batch* bt, const fpstok_params* pr,
                                                 const int32_t* start_idx, int32_t* centroid_idx,
                                                 float* centroids, int32_t* token_count,
                                                 int32_t* assign, int32_t* knn_idx, float* pooled,
                                                 int32_t* cell_count, void* stream) {
    fpstok_status st = check_tokenize(bt, pr, centroid_idx, centroids, token_count, assign,
                                      knn_idx, pooled);
    if (st != FPSTOK_OK) return st;
    if (bt->num_events == 0) return ok();
    const WorkspaceLayout L = batch_layout(bt, pr->num_patches);
    if (L.total > kNoAllocBytes)
        return fail(FPSTOK_EUNSUPPORTED,
                    "this batch needs %zu bytes of workspace; the no-allocation scratch region "
                    "holds %zu (use fpstok_tokenize with a caller workspace)",
                    L.total, kNoAllocBytes);
    hipStream_t s = (hipStream_t)stream;
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (s) {
        hipDevice_t sd = 0;
        e = hipStreamGetDevice(s, &sd);
        if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
        if ((int)sd != cur)
            return fail(FPSTOK_EINVAL, "the stream belongs to device %d, the current device is %d",
                        (int)sd, cur);
    }
    void* ws = nullptr;
    e = noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "looking up the scratch region");
    fpstok_batch staged;
    if ((st = stage_inputs(bt, staged, true, true, ws, L, s)) != FPSTOK_OK) return st;
    return run_tokenize(bt, pr, start_idx, centroid_idx, centroids, token_count, assign, knn_idx,
                        pooled, cell_count, ws, L, stream);
}

// Host-side value checks of one element of a coordinate or feature array in
// its dtype, read from the raw bits.
static bool elem_finite(const void* base, size_t i, int dtype) {
    if (dtype == FPSTOK_F32) return std::isfinite(((const float*)base)[i]);
    const uint16_t h = ((const uint16_t*)base)[i];
    // binary16: exponent bits 10..14; bfloat16: exponent bits 7..14
    return dtype == FPSTOK_F16 ? ((h >> 10) & 0x1F) != 0x1F : ((h >> 7) & 0xFF) != 0xFF;
}

static bool elem_negative(const void* base, size_t i, int dtype) {
    if (dtype == FPSTOK_F32) return ((const float*)base)[i] < 0.0f;
    const uint16_t h = ((const uint16_t*)base)[i];
    return (h & 0x8000u) != 0 && (h & 0x7FFFu) != 0;  // sign set, not -0
}

FPSTOK_API fpstok_status fpstok_validate(const fpstok_batch* bt, void* stream) {
    if (!bt) return fail(FPSTOK_EINVAL, "batch is NULL");
    const int64_t B = bt->num_events, N = bt->num_points;
    if (B < 0 || N < 0) return fail(FPSTOK_EINVAL, "negative num_events or num_points");
    if (bt->coords_dtype < FPSTOK_F32 || bt->coords_dtype > FPSTOK_BF16 ||
        bt->features_dtype < FPSTOK_F32 || bt->features_dtype > FPSTOK_BF16)
        return fail(FPSTOK_EINVAL, "unknown coords_dtype or features_dtype");
    if (B == 0) return ok();
    if (!bt->offsets) return fail(FPSTOK_EINVAL, "offsets is NULL");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    std::vector<int64_t> off((size_t)B + 1);
    e = hipMemcpy(off.data(), bt->offsets, off.size() * sizeof(int64_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy offsets");
    if (off[0] != 0) return fail(FPSTOK_EINVAL, "offsets[0] = %lld, expected 0", (long long)off[0]);
    for (int64_t b = 0; b < B; ++b)
        if (off[(size_t)b + 1] < off[(size_t)b])
            return fail(FPSTOK_EINVAL, "offsets decrease at event %lld", (long long)b);
    if (off[(size_t)B] != N)
        return fail(FPSTOK_EINVAL, "offsets[B] = %lld, expected N = %lld",
                    (long long)off[(size_t)B], (long long)N);
    if (N > 0) {
        if (!bt->coords) return fail(FPSTOK_EINVAL, "coords is NULL");
        const size_t cw = bt->coords_dtype == FPSTOK_F32 ? 4 : 2;
        std::vector<unsigned char> x((size_t)N * 4 * cw);
        e = hipMemcpy(x.data(), bt->coords, x.size(), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(e, "hipMemcpy coords");
        for (size_t q = 0; q < (size_t)N * 4; ++q)
            if (!elem_finite(x.data(), q, bt->coords_dtype))
                return fail(FPSTOK_EINVAL, "coords[%zu][%zu] is not finite", q / 4, q % 4);
        if (bt->charge_col >= 0 && bt->features && bt->num_features > bt->charge_col) {
            const int64_t C = bt->num_features;
            const size_t fw = bt->features_dtype == FPSTOK_F32 ? 4 : 2;
            std::vector<unsigned char> f((size_t)(N * C) * fw);
            e = hipMemcpy(f.data(), bt->features, f.size(), hipMemcpyDeviceToHost);
            if (e != hipSuccess) return hip_fail(e, "hipMemcpy features");
            for (int64_t i = 0; i < N; ++i) {
                const size_t q = (size_t)(i * C + bt->charge_col);
                if (!elem_finite(f.data(), q, bt->features_dtype) ||
                    elem_negative(f.data(), q, bt->features_dtype))
                    return fail(FPSTOK_EINVAL, "charge of pulse %lld is negative or not finite",
                                (long long)i);
            }
        }
    }
    return ok();
}

FPSTOK_API fpstok_status fpstok_upcast(const void* src, int64_t count, int32_t dtype,
                                       float* dst, void* stream) {
    if (count < 0) return fail(FPSTOK_EINVAL, "count must be >= 0");
    if (dtype != FPSTOK_F16 && dtype != FPSTOK_BF16)
        return fail(FPSTOK_EINVAL, "dtype must be FPSTOK_F16 or FPSTOK_BF16");
    if (count == 0) return ok();
    if (!src || !dst) return fail(FPSTOK_EINVAL, "src or dst is NULL");
    if (((uintptr_t)src & 1u) != 0 || ((uintptr_t)dst & 3u) != 0)
        return fail(FPSTOK_EINVAL, "src must be 2-byte and dst 4-byte aligned");
    const hipError_t e = launch_upcast(src, count, dtype, dst, nullptr, 0, dtype, nullptr,
                                       (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "upcast kernel launch");
    return ok();
}

FPSTOK_API fpstok_status fpstok_device_status(const void* ws, size_t ws_bytes, void* stream) {
    if (!ws) return fail(FPSTOK_EINVAL, "workspace is NULL");
    if (ws_bytes < 64 * sizeof(int32_t))
        return fail(FPSTOK_EINVAL, "workspace has %zu bytes, fewer than its header", ws_bytes);
    hipStream_t s = (hipStream_t)stream;
    int32_t word = 0;
    hipError_t e = hipMemcpyAsync(&word, (const int32_t*)ws + 3, sizeof(word),
                                  hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync of the device error word");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    if (word == 0) return ok();
    return fail(FPSTOK_EDEVICE,
                "a wait between the workgroups of one event gave up (error word 0x%x:%s%s); "
                "the outputs of the last fpstok_sample / fpstok_tokenize call on this "
                "workspace are not valid",
                (unsigned)word, (word & kErrFpsWait) ? " FPS candidate exchange" : "",
                (word & kErrPoolWait) ? " pooling partial sums" : "");
}

FPSTOK_API void fpstok_debug_set_spin_limit(uint32_t polls) {
    g_spin_limit.store(polls == 0 ? kDefaultSpinLimit : polls, std::memory_order_relaxed);
}

FPSTOK_API const char* fpstok_status_string(fpstok_status status) {
    switch (status) {
        case FPSTOK_OK: return "ok";
        case FPSTOK_EINVAL: return "invalid argument";
        case FPSTOK_EWORKSPACE: return "workspace too small";
        case FPSTOK_EUNSUPPORTED: return "unsupported";
        case FPSTOK_EHIP: return "HIP runtime error";
        case FPSTOK_EDEVICE: return "device-side failure";
    }
    return "unknown status";
}

FPSTOK_API const char* fpstok_last_error(void) { return g_last_error; }

FPSTOK_API int fpstok_version(void) { return FPSTOK_ABI_VERSION; }
