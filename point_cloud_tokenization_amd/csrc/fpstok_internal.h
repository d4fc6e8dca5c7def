// Internal interface between the C ABI (fpstok_api.cpp) and the gfx950
// kernels (fpstok_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <hip/hip_vector_types.h>
#include <stddef.h>
#include <stdint.h>

namespace fpstok {

// Pulses per chunk of the assign kernel: four threads per pulse in a
// 256-thread workgroup.
constexpr int kFpsCapPulses = 4096;  // pulses one FPS workgroup holds in registers
constexpr int kChunk = 64;

// Pulses per chunk of the chunked Voronoi pooling: the largest slot sort one
// workgroup does in LDS.
constexpr int kPoolChunk = 4096;

// A chunk of an event of more than one pooling chunk writes a record of
// per-slot float64 partial sums, and a separate combine kernel adds the
// records of each such event in chunk order: the kernel boundary publishes
// the records (no fence inside the pooling kernels).

// 64-bit words of one gang exchange record (one shard, one parity): 64
// candidate entries of one word each, the shard's bound, padding.
constexpr int kGangRecWords = 64 + 8;

// Bits of the device error word (workspace header[3]): a bounded wait
// between the workgroups of one event gave up, so that call's outputs are
// not valid.
constexpr int32_t kErrFpsWait = 1;   // the gang FPS exchange of candidate records
constexpr int32_t kErrPoolWait = 2;  // the gang shards' pooling partial sums
// Default bound on every wait between workgroups (polls; about a second).
constexpr uint32_t kDefaultSpinLimit = 1u << 22;

// Workspace carve-up.  Every region starts on a 256-byte boundary.
struct WorkspaceLayout {
    size_t header;      // int32[64]: [0] = number of chunks
    size_t chunk_ev;    // int32[max_chunks]: event of each chunk
    size_t chunk_beg;   // int32[max_chunks]: first event-local pulse of each chunk
    size_t pool_ev;     // int32[max_pool_chunks]: event of each pooling chunk
    size_t pool_beg;    // int32[max_pool_chunks]: first event-local pulse of each pooling chunk
    size_t chunk_part;  // int32[max_pool_chunks]: partial-sum record of each pooling chunk
    size_t big_ev;      // int32[2][B]: events of more than one pooling chunk and their first
                        // record
    size_t mind;        // float[N]: running min distance (large-event FPS)
    size_t near;        // int32[N]: running nearest slot (large-event FPS, no assign out)
    size_t perm;        // int32[N]: pulses sorted by token (Lloyd, pool)
    size_t item_ev;     // int32[max_items]: FPS work items (event)
    size_t item_g;      // int32[max_items]: FPS work items (shard)
    size_t gang_rec;    // uint64[max_items][2][kGangRecWords]: gang exchange records
    size_t shard_cells; // int32[max_items][P+1]: per-shard slot sizes (fused pooling)
    size_t part;        // double[max_parts][P][C+2]: partial sums per shard (fused pooling,
                        // stride C+1) or per chunk (chunked pooling, stride C+2)
    size_t coords32;    // float[N][4]: float32 copy of 16-bit coordinates (else unused)
    size_t feat32;      // float[N][C]: float32 copy of 16-bit features (else unused)
    size_t total;
    int64_t max_chunks;
    int64_t max_pool_chunks;
    int64_t max_items;
    int64_t max_parts;
};

// A gang event of n pulses has at most n / kGangPulsesPerShard shards, so
// all gangs together have at most N / kGangPulsesPerShard.  The same bound
// holds for the pooling chunks of events of more than one chunk (at most
// 2 n / kPoolChunk of them).
constexpr int64_t kGangPulsesPerShard = 2048;
static_assert(kPoolChunk >= 2 * kGangPulsesPerShard, "pooling chunks would outgrow the records");

WorkspaceLayout workspace_layout(int64_t B, int64_t N, int P, int C, int coords_dtype = 0,
                                 int features_dtype = 0);
int64_t sample_max_items(int64_t B, int64_t N);

struct SampleArgs {
    const float4* coords;
    const int64_t* offsets;
    int64_t N;
    int64_t B;
    int P;
    const int32_t* start_idx;
    int32_t* centroid_idx;
    float4* centroids;
    int32_t* token_count;
    int32_t* assign;
    float* ws_mind;
    int32_t* ws_near;
    int direct;                     // 1: item i is event i, no work list (every event
                                    // within one workgroup's registers, else streaming)
    uint32_t spin_limit;            // polls before a wait between workgroups gives up
    int32_t* header;                // [1] items, [2] claim counter, [3] device error word
                                    // (kErrFpsWait | kErrPoolWait bits), [5] gang items
                                    // (0: item i is event i)
    int32_t* item_ev;               // [max_items] event of each work item
    int32_t* item_g;                // [max_items] shard of each work item
    unsigned long long* gang_rec;   // [max_items][2][kGangRecWords] gang records
    int32_t* shard_cells;           // [max_items][P+1] per-shard slot sizes (fused pooling)
    double* gang_part;              // [gang items][P][C+1] per-shard partial sums (fused pooling)
};

struct AssignArgs {
    const float4* coords;
    const int64_t* offsets;
    int64_t N;
    int P;
    const float4* centroids;
    const int32_t* token_count;
    int32_t* assign;
    const int32_t* header;
    const int32_t* chunk_ev;
    const int32_t* chunk_beg;
    int skip_small;  // leave events with n <= P untouched
};

constexpr int kKnnMaxK = 64;  // longest kNN list (the API's FPSTOK_MAX_K)

struct KnnArgs {
    const float4* coords;
    const int64_t* offsets;
    int64_t N;
    int P;
    int k;
    const float4* centroids;
    const int32_t* token_count;
    int32_t* knn_idx;
    // with `pooled` set, each list's members are pooled by the wave that
    // ranked them (fpstok_tokenize); NULL for fpstok_knn
    const float* features;
    int C;
    int weight_col;
    float* pooled;
    int32_t* cell_count;
};

struct LloydArgs {
    const float4* coords;
    const float* features;
    const int64_t* offsets;
    int64_t N;
    int C;
    int charge_col;
    int P;
    float4* centroids;
    const int32_t* token_count;
    const int32_t* assign;
    int32_t* perm;
};

struct PoolBwdArgs {
    const float* features;
    const int64_t* offsets;
    int64_t N;
    int C;
    int wcol;  // weight column, -1: unit weights
    int P;
    int mode;  // 0 Voronoi, 1 kNN
    int k;
    const int32_t* token_count;
    const int32_t* assign;
    const int32_t* knn_idx;
    const float* pooled;
    const float* grad_pooled;
    float* grad;
    int32_t* perm;   // [N] workspace (events beyond the LDS sort)
    int64_t bits_cap;  // words of the kNN token bitmap in LDS (set by the launcher)
};

constexpr int64_t kBwdBitsCap = 24 * 1024;  // kNN backward: LDS bitmap words (96 KB)

struct PoolArgs {
    const float* features;
    const int64_t* offsets;
    int64_t N;
    int C;
    int weight_col;  // -1: unit weights
    int P;
    int k;
    const int32_t* token_count;
    const int32_t* assign;
    const int32_t* knn_idx;
    float* pooled;
    int32_t* cell_count;
    int32_t* perm;
    int32_t* header;            // chunked pooling: [4] events of > 1 chunk, [6] chunks
    const int32_t* chunk_ev;    // chunked pooling: event of each chunk
    const int32_t* chunk_beg;   // chunked pooling: first event-local pulse of each chunk
    const int32_t* chunk_part;  // chunked pooling: record of each chunk (-1: one-chunk event,
                                // -2: the event is summed whole by its first chunk)
    const int32_t* big_ev;      // chunked pooling: [m] event, [B + m] first record, m < header[4]
    int64_t B;                  // chunked pooling: events
    int whole;                  // chunked pooling: 1 when the caller's bound on event size
                                // rules out events of more than one chunk: any such event
                                // is summed whole by its first chunk (no records, no
                                // combine kernel)
    double* part;               // chunked pooling: [max_parts][P][C+2] partial sums
    int stage_cap;              // fused pooling: feature floats an event may stage in LDS
};

// Chunk list of every event, kChunk pulses per chunk (assign).
hipError_t launch_plan(const int64_t* offsets, int64_t B, int64_t N, void* ws,
                       const WorkspaceLayout& L, hipStream_t s);
// Pooling chunk list (kPoolChunk pulses per chunk, largest first), the
// chunks' partial-sum records and the list of events for the combine kernel
// (whole: every event of more than one chunk is summed by its first chunk).
hipError_t launch_plan_pool(const int64_t* offsets, int64_t B, int64_t N, void* ws,
                            const WorkspaceLayout& L, const PoolArgs& a, hipStream_t s);
hipError_t launch_sample(const SampleArgs& a, int64_t B, hipStream_t s);
// The work lists of a sample -> Lloyd (`chunks`) -> Voronoi pool (`pool`)
// sequence in one launch; then launch_sample_items runs the FPS without
// planning again.
hipError_t launch_plan_all(const SampleArgs& a, int64_t B, void* ws, const WorkspaceLayout& L,
                           const PoolArgs& pa, bool chunks, bool pool, hipStream_t s);
hipError_t launch_sample_items(const SampleArgs& a, int64_t B, hipStream_t s);
hipError_t launch_tokenize(const SampleArgs& a, const PoolArgs& pa, int64_t B, hipStream_t s);
hipError_t launch_assign(const AssignArgs& a, int64_t max_chunks, hipStream_t s);
hipError_t launch_knn(const KnnArgs& a, int64_t B, hipStream_t s);
hipError_t launch_lloyd_update(const LloydArgs& a, int64_t B, hipStream_t s);
hipError_t launch_pool_voronoi(const PoolArgs& a, int64_t max_chunks, hipStream_t s);
hipError_t launch_pool_combine(const PoolArgs& a, hipStream_t s);
hipError_t launch_pool_knn(const PoolArgs& a, int64_t B, hipStream_t s);
hipError_t launch_pack(int64_t B, int P, int D, const int32_t* tc, const float* rows,
                       float* packed, int32_t* doc_id, int32_t* cu, hipStream_t s);
hipError_t launch_unpack(int64_t B, int P, int D, const int32_t* tc, const int32_t* cu,
                         const float* packed, float* rows, hipStream_t s);
hipError_t launch_pool_backward(const PoolBwdArgs& a, int64_t B, hipStream_t s);
// Device address of this GPU's no-allocation scratch region (kNoAllocBytes
// bytes, 256-byte aligned), for the current device; looked up once per
// device, never allocated.
constexpr size_t kNoAllocBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);

// dst_a[i] = float32 value of the 16-bit src_a[i] (dtype 1: binary16, 2:
// bfloat16) for i < na, and the same for b; one launch, exact.
hipError_t launch_upcast(const void* src_a, int64_t na, int dtype_a, float* dst_a,
                         const void* src_b, int64_t nb, int dtype_b, float* dst_b, hipStream_t s);

hipError_t launch_random_start(const int64_t* offsets, int64_t B, uint64_t seed, uint64_t step,
                               int32_t* start_idx, hipStream_t s);

}  // namespace fpstok
