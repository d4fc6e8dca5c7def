/*
 * fpstok.h -- C ABI of libfpstok, the farthest-point-sampling (FPS) tokenizer
 * of the Neptune point transformer on AMD Instinct MI355X (gfx950).
 *
 * What the library computes, with the passages that define it:
 *   - An event is an irregular 4D (x, y, z, t) point cloud of pulses; FPS
 *     reduces it to at most num_patches centroids and the pulses of each
 *     token are pooled (graphnet pull request #923 "Add Neptune
 *     point-transformer backbone", section "Summary").
 *   - Small events keep one token per pulse; larger ones are reduced to
 *     centroids and pooled by Voronoi assignment or by kNN gather (same page,
 *     "What is added": FPSTokenizer).
 *   - The operation family is FPS, FPS fused with the nearest-centroid
 *     assignment, FPS with a kNN gather, and the standalone nearest
 *     assignment (same page, "What is added": farthest_point_sampling,
 *     farthest_point_sampling_with_assign, farthest_point_sampling_with_knn,
 *     nearest_assign).
 *   - FPS takes an optional start index and is always computed in float32
 *     (same page, review replies on the FPS arguments and on the removed
 *     precision argument).
 *   - Inputs: coords [N,4] with time in the fourth column, point features,
 *     per-point batch membership (README of felixyu7/neptune, "Usage"); here
 *     the batch is given as CSR offsets, events contiguous and ascending.
 *   - Tokenization = FPS down to num_patches centroids, per-token pooling by
 *     Voronoi assignment or kNN gather (assign_mode, k_neighbors), optional
 *     charge-weighted Lloyd refinement (lloyd_iters) (README, "How it works"
 *     step 1 and "Parameters").
 *   - Without a charge column every pulse has unit charge (graphnet PR #923,
 *     review reply on the no-charge case).
 *
 * Conventions fixed where the pages are silent:
 *   - squared distance d2(a,c) = ((dx*dx + dy*dy) + dz*dz) + dt*dt, each
 *     float32 operation rounded on its own (no fused multiply-add);
 *   - FPS starts at each event's first pulse unless start_idx is given; the
 *     next centroid is the not-yet-selected pulse with the largest distance
 *     to its nearest centroid, lowest pulse index on ties;
 *   - events with n <= P pass through: token t = pulse t, assign = identity,
 *     kNN list of token t = [t, -1, ...];
 *   - Voronoi ties go to the lowest token slot (FPS selection order); kNN
 *     lists ascend in (d2, pulse index);
 *   - Lloyd: per token, the charge-weighted mean of its cell accumulated in
 *     float64 in ascending pulse order and rounded to float32 (a cell with
 *     zero weight keeps its centroid), then a fresh nearest assignment;
 *     events with n <= P are not refined;
 *   - pooling: (charge-weighted) mean of all C feature columns over the
 *     token's members, float64 accumulation, float32 result, 0 for a token
 *     whose weight sum is 0;
 *   - all indices are event-local int32 (add offsets[b] for a global row);
 *     slots j >= T of an event are padded (-1 for indices, 0 for values).
 *
 * Ownership and execution:
 *   - The caller allocates and owns every buffer, including the workspace; the
 *     library allocates and frees no device memory.  Every pointer in a
 *     compute call is a device pointer unless stated otherwise.
 *   - Every compute call only enqueues work on `stream` (a hipStream_t; NULL
 *     is the legacy default stream) and returns; it makes no host-device
 *     synchronization.  Buffers must stay valid until the stream work ends.
 *   - Argument errors are found on the host before anything is enqueued and
 *     have no side effects.  Data preconditions (monotone offsets with
 *     offsets[B] = N, finite coordinates, non-negative charges, start indices
 *     in range, assignments in [0, T)) are not checked on the hot path;
 *     fpstok_validate checks them (and synchronizes).
 *   - Results are bit-identical from run to run (no floating-point atomics).
 *   - Calls on one workspace must not overlap in time (same stream, or
 *     ordered with events).  The library keeps no state between calls other
 *     than a per-device property cache.
 */
#ifndef FPSTOK_H
#define FPSTOK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FPSTOK_ABI_VERSION 3
#define FPSTOK_MAX_PATCHES 1024 /* largest num_patches accepted             */
#define FPSTOK_MAX_K 64         /* largest kNN list length accepted           */
#define FPSTOK_MAX_LLOYD 1000   /* largest lloyd_iters accepted               */

typedef enum {
    FPSTOK_OK = 0,
    FPSTOK_EINVAL = 1,      /* invalid argument; nothing was enqueued               */
    FPSTOK_EWORKSPACE = 2,  /* ws is NULL or ws_bytes < fpstok_workspace_size(...)  */
    FPSTOK_EUNSUPPORTED = 3,/* valid request beyond an implementation limit         */
    FPSTOK_EHIP = 4,        /* a HIP runtime call failed; see fpstok_last_error()   */
    FPSTOK_EDEVICE = 5      /* fpstok_device_status only: a kernel's bounded wait    */
                            /* gave up, the call's outputs are not valid             */
} fpstok_status;

typedef enum { FPSTOK_VORONOI = 0, FPSTOK_KNN = 1 } fpstok_assign_mode;

/* Element type of the coordinates or the features.  16-bit inputs are
 * upcast exactly to float32 (every binary16 and bfloat16 value is a float32
 * value) into the workspace before anything else reads them, so every result
 * equals the float32 call on the same values: FPS and every sum stay in
 * float32 / float64.  (Pull Request #923, "Add Neptune point-transformer
 * backbone": its "What is added" list has low-precision tests, and the review
 * thread on the FPS precision argument settles that FPS runs in float32 on
 * both backends whatever the input dtype.)  Gradients (fpstok_pool_backward)
 * are float32 whatever the features' dtype. */
typedef enum { FPSTOK_F32 = 0, FPSTOK_F16 = 1, FPSTOK_BF16 = 2 } fpstok_dtype;

/* One CSR batch of events.  All pointers are device pointers. */
typedef struct {
    const void* coords;      /* [N,4] row-major (x,y,z,t), coords_dtype; 16-byte  */
                             /* aligned for float32, 8-byte for 16-bit types      */
    const void* features;    /* [N,C] row-major, features_dtype; aligned to its   */
                             /* element; may be NULL for calls that do not read   */
                             /* features                                          */
    const int64_t* offsets;  /* [B+1] int64: event b is rows offsets[b] ..        */
                             /* offsets[b+1]-1; offsets[0]=0, offsets[B]=N         */
    int64_t num_events;      /* B >= 0                                            */
    int64_t num_points;      /* N >= 0, N < 2^31                                  */
    int32_t num_features;    /* C >= 1 for calls that read features                */
    int32_t charge_col;      /* charge column 0..C-1, or -1 for unit charge       */
    int64_t max_event_points;/* optional host-side bound on the pulses of any     */
                             /* event, 0 if unknown.  A bound <= 4096 lets        */
                             /* fpstok_sample / fpstok_tokenize skip planning     */
                             /* their work list (every event then runs on one     */
                             /* workgroup); a bound that is too small stays       */
                             /* correct: a larger event falls back to the slower  */
                             /* one-workgroup streaming FPS.                      */
    int32_t coords_dtype;    /* fpstok_dtype of coords (FPSTOK_F32 = 0)           */
    int32_t features_dtype;  /* fpstok_dtype of features (FPSTOK_F32 = 0); with a */
                             /* 16-bit type the workspace also holds the float32  */
                             /* copy (fpstok_workspace_size counts it)            */
} fpstok_batch;

typedef struct {
    int32_t num_patches;     /* P: 1..FPSTOK_MAX_PATCHES                          */
    int32_t k;               /* kNN list length 1..FPSTOK_MAX_K (kNN mode only)   */
    int32_t lloyd_iters;     /* L: 0..FPSTOK_MAX_LLOYD                            */
    int32_t assign_mode;     /* FPSTOK_VORONOI or FPSTOK_KNN                      */
    int32_t pool_weighted;   /* 0: plain mean; 1: charge-weighted mean            */
} fpstok_params;

/* Bytes of device workspace every compute call of this batch shape needs
 * (depends on B, N, num_patches, num_features and the input dtypes; params
 * may be NULL for the largest num_patches).  Host-only; never fails; 0 for
 * B = 0. */
size_t fpstok_workspace_size(const fpstok_batch* batch, const fpstok_params* params);

/* FPS of every event (farthest_point_sampling / _with_assign).  For n > P:
 * P centroids by FPS from start_idx[b] (NULL: 0); for n <= P: pass-through.
 *   start_idx    [B] int32 event-local start pulse, or NULL (device)
 *   centroid_idx [B,P] int32 out: selected pulse of each slot, -1 padded
 *   centroids    [B,P,4] f32 out: coordinates of each slot, 0 padded
 *   token_count  [B] int32 out: T = min(n, P)
 *   assign       [N] int32 out: Voronoi slot of every pulse (the fused
 *                nearest-centroid assignment), or NULL to skip it
 * Errors: EINVAL (NULL coords/offsets/outputs, misaligned coords, bad P),
 * EWORKSPACE, EUNSUPPORTED (N >= 2^31), EHIP. */
fpstok_status fpstok_sample(const fpstok_batch* batch, const fpstok_params* params,
                            const int32_t* start_idx, int32_t* centroid_idx, float* centroids,
                            int32_t* token_count, int32_t* assign, void* ws, size_t ws_bytes,
                            void* stream);

/* Standalone nearest-centroid assignment (nearest_assign) of every pulse of
 * every event to the event's first token_count[b] centroids, lowest slot on
 * ties.  This is the plain argmin for every event, pass-through ones included.
 *   centroids   [B,P,4] f32 in;  token_count [B] int32 in (T >= 1 if n >= 1)
 *   assign      [N] int32 out
 * Errors: EINVAL, EWORKSPACE, EUNSUPPORTED, EHIP. */
fpstok_status fpstok_assign(const fpstok_batch* batch, const fpstok_params* params,
                            const float* centroids, const int32_t* token_count, int32_t* assign,
                            void* ws, size_t ws_bytes, void* stream);

/* kNN gather (farthest_point_sampling_with_knn, assign_mode="knn"): for every
 * event with n > P and every slot j < token_count[b], the min(k, n) pulses
 * with the smallest (d2(pulse, centroid_j), pulse index), ascending, -1
 * padded; pass-through events get [t, -1, ...]; slots j >= T are all -1.
 *   centroids [B,P,4] f32 in; token_count [B] int32 in
 *   knn_idx   [B,P,k] int32 out
 * Errors: EINVAL (k out of range ...), EWORKSPACE, EUNSUPPORTED, EHIP. */
fpstok_status fpstok_knn(const fpstok_batch* batch, const fpstok_params* params,
                         const float* centroids, const int32_t* token_count, int32_t* knn_idx,
                         void* ws, size_t ws_bytes, void* stream);

/* params->lloyd_iters rounds of charge-weighted Lloyd refinement on every
 * event with n > P (others untouched): the neptune README, "How it works"
 * (the refinement step of the tokenizer) and "Parameters" (lloyd_iters).
 * Reads the features' charge column (unit charge if charge_col = -1: Pull
 * Request #923, review reply on events without a charge column).
 *   centroids [B,P,4] f32 in/out; token_count [B] int32 in
 *   assign    [N] int32 in/out (Voronoi slots, e.g. from fpstok_sample)
 * L = 0 is a no-op.  Errors: EINVAL, EWORKSPACE, EUNSUPPORTED, EHIP. */
fpstok_status fpstok_lloyd(const fpstok_batch* batch, const fpstok_params* params,
                           float* centroids, const int32_t* token_count, int32_t* assign,
                           void* ws, size_t ws_bytes, void* stream);

/* Per-token pooling of the features (Pull Request #923, "Summary": the
 * pulses of each token are pooled; the neptune README, "How it works").
 * Voronoi mode: the members of slot j are the pulses with assign = j; kNN
 * mode: the entries != -1 of knn_idx[b][j].  Weight = charge if
 * params->pool_weighted and charge_col >= 0, else 1.
 *   assign     [N] int32 in (Voronoi mode; may be NULL in kNN mode)
 *   knn_idx    [B,P,k] int32 in (kNN mode; may be NULL in Voronoi mode)
 *   pooled     [B,P,C] f32 out, 0 for j >= T and for zero-weight tokens
 *   cell_count [B,P] int32 out: members per slot (may be NULL)
 * Errors: EINVAL, EWORKSPACE, EUNSUPPORTED, EHIP. */
fpstok_status fpstok_pool(const fpstok_batch* batch, const fpstok_params* params,
                          const int32_t* token_count, const int32_t* assign,
                          const int32_t* knn_idx, float* pooled, int32_t* cell_count, void* ws,
                          size_t ws_bytes, void* stream);

/* The whole tokenizer in one call: fpstok_sample, then fpstok_lloyd
 * (lloyd_iters > 0), fpstok_knn (kNN mode), fpstok_pool, with the same
 * results as calling them in that order (README of felixyu7/neptune, "How it
 * works" step 1: FPS, Voronoi or kNN pooling, optional Lloyd).  In Voronoi mode without Lloyd the
 * FPS and the pooling run in one kernel: each workgroup pools its event as
 * soon as its sampling ends; in kNN mode each token's list is pooled by the
 * wave that ranked it, in the kNN kernel.  Outputs as in the calls above; `assign` is
 * required in Voronoi mode and for Lloyd (else it may be NULL), `knn_idx` in
 * kNN mode (else it may be NULL), `features` are always read.
 * Errors: those of the calls it makes. */
fpstok_status fpstok_tokenize(const fpstok_batch* batch, const fpstok_params* params,
                              const int32_t* start_idx, int32_t* centroid_idx, float* centroids,
                              int32_t* token_count, int32_t* assign, int32_t* knn_idx,
                              float* pooled, int32_t* cell_count, void* ws, size_t ws_bytes,
                              void* stream);

/* For callers that cannot allocate device memory (code under HIP graph or
 * stream capture, tight serving loops, harnesses that forbid allocation):
 * fpstok_tokenize with the same arguments and results, but no workspace.
 * Its workspace is a fixed scratch region of FPSTOK_NOALLOC_MAX_WORKSPACE
 * bytes in the library's device memory, one per GPU, held by every GPU the
 * library runs on until the process ends; the call allocates and frees
 * nothing.  Every call on one GPU uses that GPU's region (the kernels leave
 * in it what the last call wrote and clear what must start at zero), so calls
 * that overlap in time on one GPU -- from several streams or host threads --
 * race and must be serialized by the caller.  `stream` must belong to the
 * current device (NULL: the legacy default stream).
 * Errors: as fpstok_tokenize; EUNSUPPORTED when the batch needs more than
 * FPSTOK_NOALLOC_MAX_WORKSPACE bytes of workspace (fpstok_workspace_size;
 * nothing is enqueued); EINVAL when the stream is on another device. */
#define FPSTOK_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
fpstok_status fpstok_tokenize_noalloc(const fpstok_batch* batch, const fpstok_params* params,
                                      const int32_t* start_idx, int32_t* centroid_idx,
                                      float* centroids, int32_t* token_count, int32_t* assign,
                                      int32_t* knn_idx, float* pooled, int32_t* cell_count,
                                      void* stream);

/* ------------------------------------------------ next to the path -- */

/* Packing of every event's tokens into one variable-length sequence for
 * block-diagonal attention (graphnet PR #923, "What is added":
 * models/utils.py pack / unpack for variable-length packing; its review
 * thread: doc_id is the event index of every packed token, the packed length
 * is the number of tokens).  Event b contributes its first T_b =
 * token_count[b] slots, events in order.
 *   token_count [B] int32 in (T_b outside [0, P] is clamped into it)
 *   rows        [B,P,D] f32 in: one row of D floats per slot (pooled
 *               features, D = C; centroids, D = 4; ...)
 *   packed      [B*P, D] f32 out: rows 0 .. n_tokens-1 receive the tokens'
 *               rows, event after event; later rows are not written
 *   doc_id      [B*P] int32 out: event of every packed row (same extent), or
 *               NULL
 *   cu_seqlens  [B+1] int32 out: cu_seqlens[b] = T_0 + ... + T_{b-1};
 *               cu_seqlens[B] = n_tokens
 * No workspace.  Errors: EINVAL (NULL pointers, num_events < 0, num_patches
 * outside [1, FPSTOK_MAX_PATCHES], row_width < 1), EUNSUPPORTED (B*P >= 2^31),
 * EHIP. */
fpstok_status fpstok_pack(int64_t num_events, int32_t num_patches, int32_t row_width,
                          const int32_t* token_count, const float* rows, float* packed,
                          int32_t* doc_id, int32_t* cu_seqlens, void* stream);

/* The inverse of fpstok_pack: rows[b][j] = packed[cu_seqlens[b] + j] for
 * j < T_b, 0 for T_b <= j < P.
 *   token_count [B] int32 in (clamped into [0, P]); cu_seqlens [B+1] int32 in
 *   (as fpstok_pack writes it); packed [n_tokens, D] f32 in;
 *   rows [B,P,D] f32 out
 * Errors: as fpstok_pack. */
fpstok_status fpstok_unpack(int64_t num_events, int32_t num_patches, int32_t row_width,
                            const int32_t* token_count, const int32_t* cu_seqlens,
                            const float* packed, float* rows, void* stream);

/* Gradient of fpstok_pool with respect to the features, for training through
 * the tokenizer (graphnet PR #923, "Dependencies": time per training step;
 * "What is added": gradient tests).  Token j of event b with members M_j
 * (Voronoi: assign = j; kNN: the list entries != -1), weights w_i, weight sum
 * W_j and forward output m_j = pooled[b][j]: for i in M_j and W_j != 0
 *   d m_j[c] / d f_i[c'] = [c = c'] w_i / W_j
 *                        + [c' = weight column] (f_i[c] - m_j[c]) / W_j
 * (the second term only for weighted pooling with charge_col >= 0; a token of
 * zero weight contributes nothing).  grad_features[i][c'] = sum over the
 * tokens j containing i, ascending, of sum_c grad_pooled[b][j][c] *
 * d m_j[c] / d f_i[c'], accumulated in float64 in that order (per token:
 * grad_pooled[j][c'] * w_i / W_j, then, for the weight column,
 * (sum over c ascending of grad_pooled[j][c] * (f_i[c] - m_j[c])) / W_j),
 * with W_j the float64 weight sum in member order; rounded to float32.
 * Pulses in no token get 0.
 *   token_count [B] int32 in; assign [N] int32 in (Voronoi mode) or knn_idx
 *   [B,P,k] int32 in (kNN mode), as given to fpstok_pool
 *   pooled      [B,P,C] f32 in: the output of fpstok_pool
 *   grad_pooled [B,P,C] f32 in (rows j >= T_b are ignored)
 *   grad_features [N,C] f32 out
 * Errors: as fpstok_pool. */
fpstok_status fpstok_pool_backward(const fpstok_batch* batch, const fpstok_params* params,
                                   const int32_t* token_count, const int32_t* assign,
                                   const int32_t* knn_idx, const float* pooled,
                                   const float* grad_pooled, float* grad_features, void* ws,
                                   size_t ws_bytes, void* stream);

/* A random FPS start per event, for FPS's random_start option (graphnet PR
 * #923, review thread on the FPS arguments: start_idx, random_start,
 * generator; the pages do not say how the start is drawn).  Event b takes
 * word 0 of Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random
 * Numbers: As Easy as 1, 2, 3", SC 2011) at counter (b low, b high, step low,
 * step high) with key (seed low, seed high), maps it to
 * floor(u * n_b / 2^32), a pulse index in [0, n_b), and writes it to
 * start_idx[b] (0 for an empty event).  Pass the result as start_idx to
 * fpstok_sample or fpstok_tokenize; change `step` (e.g. per training step)
 * for new draws with the same seed.
 *   offsets   [B+1] int64 in (device); start_idx [B] int32 out (device)
 * Errors: EINVAL (NULL pointers, num_events < 0), EHIP. */
fpstok_status fpstok_random_start(const int64_t* offsets, int64_t num_events, uint64_t seed,
                                  uint64_t step, int32_t* start_idx, void* stream);

/* Device-side status of the last fpstok_sample or fpstok_tokenize call on
 * the workspace `ws` (its first ws_bytes bytes; at least the 256-byte
 * header).  An event of more than 4096 pulses is split over a gang of
 * workgroups that wait for one another's candidate records and pooling
 * partial sums; every such wait is bounded (a few million polls) so that a
 * stalled partner can never hang the GPU.  A wait that gives up sets a word
 * in the workspace and the call completes with outputs that are not valid.
 * This function waits for `stream` (it synchronizes: not for the hot path),
 * reads that word and returns FPSTOK_OK, or FPSTOK_EDEVICE with the detail
 * in fpstok_last_error(), or FPSTOK_EHIP.  Every fpstok_sample and
 * fpstok_tokenize call clears the word when it starts; the other calls
 * neither set nor clear it.  Errors: EINVAL (NULL ws, ws_bytes < 256). */
fpstok_status fpstok_device_status(const void* ws, size_t ws_bytes, void* stream);

/* Testing only: the number of polls after which a wait between workgroups
 * gives up, for calls made after this one in the process (0 restores the
 * default).  Tests of the failure path set a tiny limit so that a gang's
 * wait gives up and fpstok_device_status reports it, while every kernel still
 * ends normally.  Not for production use: a small limit makes large events
 * fail. */
void fpstok_debug_set_spin_limit(uint32_t polls);

/* Debug check of the data preconditions of `batch` (offsets monotone with
 * offsets[0] = 0 and offsets[B] = N, finite coords, charge >= 0 when
 * charge_col >= 0).  Copies the inputs to the host and synchronizes `stream`:
 * not for the hot path.  Returns FPSTOK_OK or FPSTOK_EINVAL (the reason is in
 * fpstok_last_error()), or FPSTOK_EHIP. */
fpstok_status fpstok_validate(const fpstok_batch* batch, void* stream);

/* dst[i] = the float32 value of src[i] for i < count, src of dtype
 * FPSTOK_F16 (IEEE binary16, subnormals kept) or FPSTOK_BF16 (bfloat16:
 * the upper 16 bits of a float32).  The conversion every call above applies
 * to 16-bit inputs, exposed for callers that convert once and reuse the
 * float32 copy.  Exact for every finite and infinite value; a NaN stays a
 * NaN of the same sign (a signalling binary16 NaN may come back quiet).
 * src 2-byte aligned, dst 4-byte aligned, device pointers; count >= 0;
 * enqueued on `stream`; EINVAL for a NULL pointer with count > 0, another
 * dtype or misalignment. */
fpstok_status fpstok_upcast(const void* src, int64_t count, int32_t dtype, float* dst,
                            void* stream);

/* Static description of a status code. */
const char* fpstok_status_string(fpstok_status status);

/* Detail of the last failed call on this host thread ("" if none). */
const char* fpstok_last_error(void);

/* FPSTOK_ABI_VERSION of the library. */
int fpstok_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FPSTOK_H */
