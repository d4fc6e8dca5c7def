// gfx950 kernels of libfpstok: the FPS tokenizer of the Neptune point
// transformer (graphnet pull request #923 "Add Neptune point-transformer
// backbone", "What is added"; README of felixyu7/neptune, "How it works").
//
// Wave64 throughout.  No MFMA: the only contraction is 4 wide and the
// distance must be the exact float32 sum ((dx^2+dy^2)+dz^2)+dt^2, so every
// hot loop is plain VALU.  No floating-point atomics anywhere: every float64
// sum runs in a fixed order, so results are bit-identical run to run.
//
// Every kernel clamps the CSR offsets into [0, N] and ignores out-of-range
// slot or pulse indices, so malformed inputs give wrong numbers, never an
// out-of-bounds access.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "fpstok_internal.h"

namespace fpstok {

// ------------------------------------------------------------ device helpers

// Squared 4D distance, fixed axis order, each operation rounded on its own
// (the file is compiled with -ffp-contract=off).
__device__ __forceinline__ float sqd(float px, float py, float pz, float pt, float cx, float cy,
                                     float cz, float ct) {
    float dx = px - cx;
    float dy = py - cy;
    float dz = pz - cz;
    float dt = pt - ct;
    float r = dx * dx;
    r = r + dy * dy;
    r = r + dz * dz;
    r = r + dt * dt;
    return r;
}

__device__ __forceinline__ void event_range(const int64_t* offsets, int64_t N, int64_t b,
                                            int64_t& off, int& n) {
    int64_t lo = offsets[b];
    int64_t hi = offsets[b + 1];
    lo = lo < 0 ? 0 : (lo > N ? N : lo);
    hi = hi < lo ? lo : (hi > N ? N : hi);
    off = lo;
    n = (int)(hi - lo);
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Workgroup barrier that orders LDS accesses only: it waits for this wave's
// LDS operations but leaves its global loads and stores in flight (a plain
// __syncthreads also drains those).  For code whose threads communicate
// through LDS alone.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// number of set bits of m in lanes below this one
__device__ __forceinline__ int mbcnt(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float readlane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// v permuted across lanes by a DPP control; lanes of rows outside ROW_MASK
// get `identity`.  Passing the identity of the combining operation lets the
// compiler fold the move into the ALU instruction (v_max_i32_dpp, ...).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int v, int identity) {
    return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROW_MASK, 0xF, false);
}

// DPP controls (gfx9 family): quad permutes, row mirrors, row broadcasts.
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowMirror = 0x140;
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;

// Wave-wide minimum / maximum, returned uniformly: four in-row DPP steps,
// then the two row broadcasts that carry the result into lane 63.
__device__ __forceinline__ int wave_min_i(int v) {
    constexpr int I = INT32_MAX;
    v = min(v, dpp_i<kQuadSwap1, 0xF>(v, I));
    v = min(v, dpp_i<kQuadSwap2, 0xF>(v, I));
    v = min(v, dpp_i<kRowHalfMirror, 0xF>(v, I));
    v = min(v, dpp_i<kRowMirror, 0xF>(v, I));
    v = min(v, dpp_i<kRowBcast15, 0xA>(v, I));
    v = min(v, dpp_i<kRowBcast31, 0xC>(v, I));
    return readlane_i(v, 63);
}

__device__ __forceinline__ int wave_max_i(int v) {
    constexpr int I = INT32_MIN;
    v = max(v, dpp_i<kQuadSwap1, 0xF>(v, I));
    v = max(v, dpp_i<kQuadSwap2, 0xF>(v, I));
    v = max(v, dpp_i<kRowHalfMirror, 0xF>(v, I));
    v = max(v, dpp_i<kRowMirror, 0xF>(v, I));
    v = max(v, dpp_i<kRowBcast15, 0xA>(v, I));
    v = max(v, dpp_i<kRowBcast31, 0xC>(v, I));
    return readlane_i(v, 63);
}

// Inclusive prefix sum over the wave (every lane active) with DPP: shifts of
// 1, 2, 4 and 8 lanes inside each row of 16 (lanes without a source add 0),
// then the row totals carried into the later rows by the two row
// broadcasts.  No LDS round trips.
constexpr int kRowShr1 = 0x111;
constexpr int kRowShr2 = 0x112;
constexpr int kRowShr4 = 0x114;
constexpr int kRowShr8 = 0x118;
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, kRowShr1, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kRowShr2, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kRowShr4, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kRowShr8, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return v;
}

// Lowest pulse index not yet selected, from a per-lane 32-bit slice of the
// selection bitmap (lane l holds indices 32l .. 32l+31).  The caller
// guarantees such an index exists below 2048.
__device__ __forceinline__ int first_unselected(uint32_t selbits) {
    uint32_t inv = ~selbits;
    uint64_t bl = ballot(inv != 0u);
    int L = (int)__builtin_ctzll(bl);
    uint32_t w = (uint32_t)readlane_i((int)inv, L);
    return L * 32 + (int)__builtin_ctz(w);
}

__device__ __forceinline__ void mark_selected(uint32_t& selbits, int s) {
    if (s < 2048 && lane_id() == (s >> 5)) selbits |= 1u << (s & 31);
}

// ------------------------------------------------------------------- planner

// One workgroup of 1024 threads: split every event into chunks of kChunk
// pulses (an empty event gets one chunk so per-event work still runs) and
// write the chunk list.
__device__ __forceinline__ void plan_chunks(const int64_t* __restrict__ offsets,
                                                    int64_t B, int64_t N, int64_t max_chunks,
                                                    int32_t* __restrict__ header,
                                                    int32_t* __restrict__ chunk_ev,
                                                    int32_t* __restrict__ chunk_beg) {
    __shared__ int s_wsum[16];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    int carry = 0;
    for (int64_t base = 0; base < B; base += 1024) {
        const int64_t b = base + tid;
        int nch = 0;
        if (b < B) {
            int64_t off;
            int n;
            event_range(offsets, N, b, off, n);
            nch = n > 0 ? (n + kChunk - 1) / kChunk : 1;
        }
        int incl = wave_incl_scan(nch);
        if (lane == 63) s_wsum[wave] = incl;
        __syncthreads();
        int wbase = 0, total = 0;
        for (int w = 0; w < 16; ++w) {
            int v = s_wsum[w];
            if (w < wave) wbase += v;
            total += v;
        }
        // malformed (overlapping) offsets can ask for more chunks than the
        // list holds; those are dropped rather than written out of bounds
        const int64_t pos = (int64_t)carry + wbase + incl - nch;
        for (int c = 0; c < nch && pos + c < max_chunks; ++c) {
            chunk_ev[pos + c] = (int32_t)b;
            chunk_beg[pos + c] = c * kChunk;
        }
        carry = (int)min((int64_t)carry + total, max_chunks);
        __syncthreads();
    }
    if (tid == 0) header[0] = carry;
}

constexpr int kTailBuckets = 32;  // length bands of the partial chunks
static_assert(kPoolChunk % kTailBuckets == 0 && kTailBuckets <= 64, "tail bands");

// The pooling chunk list (kPoolChunk pulses per chunk), one workgroup of
// 1024 threads, longest first: every event's full chunks, then every event's
// last, partial chunk (an empty event gets one empty chunk).  In the kBands
// form, when the list is longer than band_over (the workers that take it in
// rounds), the partial chunks go by length in kTailBuckets bands of
// decreasing length (a band's chunks in any order: a chunk's output does not
// depend on its place in the list), so that the rounds give the workers even
// loads; otherwise, and always in the other form, in event order (the other
// form has no band code: it serves the lists that fit one round, where the
// planner's own time is what counts).  The chunks of an event of
// more than one chunk get consecutive partial-sum records (-1: the event is
// one chunk) and the event is listed in big_ev with its first record for the
// combine kernel (count in header[4]; the chunk count goes to header[6]).
// With `whole`, an event of more than one chunk gets no records instead and
// is marked -2: summed whole by its first chunk.
// Malformed (overlapping) offsets can ask for more chunks or records than
// the lists hold: extra chunks are dropped, an event without room for its
// records is marked -2 too, and a listed event without room is listed as -1;
// nothing is written out of bounds.
template <bool kBands>
__device__ __forceinline__ void plan_pool(const int64_t* __restrict__ offsets,
                                                         int64_t B, int64_t N, int64_t max_chunks,
                                                         int64_t max_parts,
                                                         int32_t* __restrict__ header,
                                                         int32_t* __restrict__ chunk_ev,
                                                         int32_t* __restrict__ chunk_beg,
                                                         int32_t* __restrict__ chunk_part,
                                                         int32_t* __restrict__ big_ev,
                                                         int whole, int64_t band_over) {
    __shared__ int s_sum[3][16];
    __shared__ int s_tt;                // all partial chunks
    __shared__ int s_tb[kTailBuckets];  // tails per band, then each band's first list place
    __shared__ int s_tc[kTailBuckets];  // places taken in each band
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    if constexpr (kBands) {
        if (tid < kTailBuckets) {
            s_tb[tid] = 0;
            s_tc[tid] = 0;
        }
        __syncthreads();
    }
    int64_t carry = 0, tail0 = 0;
    bool banded = false;
    int bcarry = 0;
    int n_first = 0;  // the size of event tid, kept from the first pass
    for (int pass = 0; pass < 2; ++pass) {
        int64_t pcarry = 0;
        if (kBands && pass == 1) {
            // band places: an exclusive scan of the band counts (band 0: the
            // longest tails)
            if (wave == 0) {
                const int v = lane < kTailBuckets ? s_tb[lane] : 0;
                const int incl = wave_incl_scan(v);
                if (lane < kTailBuckets) s_tb[lane] = incl - v;
                if (lane == 63) s_tt = incl;
            }
            __syncthreads();
            tail0 = carry;
            banded = carry + s_tt > band_over;
        }
        for (int64_t base = 0; base < B; base += 1024) {
            const int64_t b = base + tid;
            int nf = 0, tl = 0, band = 0;
            if (b < B) {
                int n;
                if (pass == 1 && base == 0) {
                    n = n_first;
                } else {
                    int64_t off;
                    event_range(offsets, N, b, off, n);
                    if (base == 0) n_first = n;
                }
                nf = n / kPoolChunk;
                tl = n % kPoolChunk != 0 || n == 0 ? 1 : 0;
                band = (kPoolChunk - 1 - n % kPoolChunk) / (kPoolChunk / kTailBuckets);
                if (kBands && pass == 0 && tl) atomicAdd(&s_tb[band], 1);
            }
            const int nch = nf + tl;
            const int cnt = pass == 0 ? nf : tl;  // chunks this pass places
            const int np = nch > 1 && !whole ? nch : 0;
            const int nb = pass == 0 && np > 0 ? 1 : 0;
            const int v[3] = {cnt, np, nb};
            int incl[3], pre[3] = {0, 0, 0}, tot[3] = {0, 0, 0};
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                incl[q] = wave_incl_scan(v[q]);
                if (lane == 63) s_sum[q][wave] = incl[q];
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 3; ++q)
                for (int w = 0; w < 16; ++w) {
                    const int x = s_sum[q][w];
                    pre[q] += w < wave ? x : 0;
                    tot[q] += x;
                }
            const int64_t pos = kBands && pass == 1 && banded
                                    ? (cnt ? tail0 + s_tb[band] + atomicAdd(&s_tc[band], 1)
                                           : (int64_t)0)
                                    : carry + pre[0] + incl[0] - cnt;
            const int64_t ppos = pcarry + pre[1] + incl[1] - np;
            const bool room = ppos + np <= max_parts;
            for (int c = 0; c < cnt && pos + c < max_chunks; ++c) {
                const int k = pass == 0 ? c : nf;  // chunk number inside the event
                chunk_ev[pos + c] = (int32_t)b;
                chunk_beg[pos + c] = k * kPoolChunk;
                chunk_part[pos + c] = nch == 1 ? -1 : (room && !whole ? (int)(ppos + k) : -2);
            }
            if (nb) {
                const int m = bcarry + pre[2] + incl[2] - 1;
                big_ev[m] = room ? (int32_t)b : -1;
                big_ev[B + m] = (int32_t)ppos;
            }
            carry = min(carry + tot[0], max_chunks);
            pcarry += tot[1];
            bcarry += tot[2];
            __syncthreads();
        }
    }
    if (tid == 0) {
        header[4] = bcarry;
        header[6] = (int)carry;
    }
}

__global__ __launch_bounds__(1024) void plan_kernel(const int64_t* __restrict__ offsets, int64_t B,
                                                    int64_t N, int64_t max_chunks,
                                                    int32_t* __restrict__ header,
                                                    int32_t* __restrict__ chunk_ev,
                                                    int32_t* __restrict__ chunk_beg) {
    plan_chunks(offsets, B, N, max_chunks, header, chunk_ev, chunk_beg);
}

template <bool kBands>
__global__ __launch_bounds__(1024) void plan_pool_kernel(const int64_t* __restrict__ offsets,
                                                         int64_t B, int64_t N, int64_t max_chunks,
                                                         int64_t max_parts,
                                                         int32_t* __restrict__ header,
                                                         int32_t* __restrict__ chunk_ev,
                                                         int32_t* __restrict__ chunk_beg,
                                                         int32_t* __restrict__ chunk_part,
                                                         int32_t* __restrict__ big_ev, int whole,
                                                         int64_t band_over) {
    plan_pool<kBands>(offsets, B, N, max_chunks, max_parts, header, chunk_ev, chunk_beg,
                      chunk_part, big_ev, whole, band_over);
}

// ---------------------------------------------------------------------- FPS

#define FPSTOK_MAX_SLOTS 1024
constexpr int kFpsT = 256;                 // threads per workgroup (4 waves)
constexpr int kFpsW = kFpsT / 64;
constexpr int kFpsM = 16;                  // register-resident pulses per thread
constexpr int kFpsCap = kFpsT * kFpsM;     // pulses one workgroup holds in registers
static_assert(kFpsCap == kFpsCapPulses, "host and device disagree on the register capacity");
constexpr int kGangMax = 64;               // workgroups sharing one event at most

struct __align__(16) FpsSlot {
    float v;
    int i;
    float pad0, pad1;
    float4 c;
};

// The part of an event one workgroup holds.  A gang is the set of G
// workgroups that share one event; each keeps a contiguous shard of pulses in
// registers, and the shards exchange candidates through records in device
// memory.
struct Shard {
    int lo;                    // first event-local pulse of the shard
    int cnt;                   // pulses in the shard
    int g;                     // shard index
    int G;                     // shards of the event
    unsigned long long* rec;   // records of the gang: [G][2][kGangRecWords]
    int32_t* err;              // device error word (bounded wait exceeded)
    uint32_t spin_limit;       // polls before a wait gives up
};


// Write the selection order (and the selected coordinates) of one event.
__device__ __forceinline__ void write_selection(const SampleArgs& a, int64_t b,
                                                const float4* __restrict__ p, const int* s_sel) {
    lds_barrier();
    for (int j = threadIdx.x; j < a.P; j += blockDim.x) {
        const int s = s_sel[j];
        a.centroid_idx[b * a.P + j] = s;
        a.centroids[b * a.P + j] = p[s];
    }
}

// ------------------------------------ single-workgroup FPS, candidate list

constexpr int kBmW4 = 8;  // 128-bit words per bitmap row: events of up to 1024 pulses
constexpr int kStage = 6144;              // feature floats an event may stage in LDS
constexpr int kStageR = kStage / kFpsT;   // staged floats per thread

// Feature rows of a single-workgroup event, copied to LDS while its FPS
// runs (nf = 0: none).  The loads are issued once the pulses are in
// registers; the FPS loop itself issues no global loads, so they complete
// in its shadow and are written to `dst` after the last iteration, followed
// by one all-zero row (the padding row of the pooling sums).
struct Stage {
    const float* src;  // the event's first feature row
    int nf;            // floats to copy (n * C), at most kStage - C
    int nz;            // floats written: nf + C (the zero row), 0 when none
    float* dst;        // LDS, kStage floats
    int defer_sel;     // 1: the caller writes the selection (centroid_idx, centroids)
};

constexpr int kListCap = 64;  // entries of the candidate list (one per lane)
constexpr int kNoEntry = (int)0xBF800000;  // bit pattern of -1.0f: an empty entry

// LDS of a single-workgroup FPS.  The offers of an exchange are
// double-buffered by exchange parity: a wave that runs ahead into the next
// exchange writes the other buffer, and one exchange later every wave has
// passed a barrier after its last read of this one.
struct SingleLds {
    int ov[2][kFpsW][64];      // offered distances (float bits), in lane order per wave
    int oi[2][kFpsW][64];      // offered pulse indices
    float4 oc[2][kFpsW][64];   // offered coordinates
    int4 wc[2];                // offers of each wave
    int4 wb[2];                // bound of each wave
    FpsSlot list[kListCap];    // the kept list when the offers do not fit one
    int wd[kFpsW];             // each wave's largest kept entry left out of a full list
    uint32_t bm[kFpsW][64];    // per-wave selection bitmap (degenerate case only)
};

static_assert(offsetof(SingleLds, ov) == 0 && offsetof(SingleLds, oi) == 2048 &&
                  offsetof(SingleLds, oc) == 4096 && offsetof(SingleLds, wc) == 12288 &&
                  offsetof(SingleLds, wb) == 12320,
              "the hand-scheduled exchange addresses this layout");

// LDS of a shard's own exchange in the gang FPS.
struct FpsLds {
    FpsSlot wl[kFpsW][64];    // each wave's contribution to an exchange
    FpsSlot list[kListCap];   // the workgroup's new candidate list
    int wc[kFpsW];            // entries of each wave's contribution
    int wb[kFpsW];            // each wave's bound
    int wd[kFpsW];            // each wave's largest offer left out of a full list
    uint32_t bm[kFpsW][64];   // per-wave selection bitmap (degenerate case only)
};

// Lowest pulse index that no iteration 0..j has selected (the caller knows
// one exists below 2048).  Selections 0 .. 64*(j/64)-1 are in s_sel; those
// of the current block of 64 are in `selv` (lane q: iteration 64*(j/64)+q).
// Built per wave in LDS with atomic ORs; used only when every pulse has
// minimum distance 0.
__device__ __forceinline__ int first_unselected_lds(uint32_t* bm, const int* s_sel, int selv,
                                                    int j) {
    const int lane = lane_id();
    bm[lane] = 0u;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    const int blk = j & ~63;
    for (int q = lane; q < blk; q += 64) {
        const int v = s_sel[q];
        if (v >= 0 && v < 2048) atomicOr(&bm[v >> 5], 1u << (v & 31));
    }
    if (lane <= (j & 63) && selv >= 0 && selv < 2048) atomicOr(&bm[selv >> 5], 1u << (selv & 31));
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    return first_unselected(bm[lane]);
}

// Lowest pulse index that no iteration 0..j has selected (the caller knows
// one exists below 2048); s_sel[0..j] holds those selections.  Built per
// wave in LDS with atomic ORs; used only when every pulse has minimum
// distance 0.
__device__ __forceinline__ int first_unselected_sel(uint32_t* bm, const int* s_sel, int j) {
    const int lane = lane_id();
    bm[lane] = 0u;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    for (int q = lane; q <= j; q += 64) {
        const int v = s_sel[q];
        if (v >= 0 && v < 2048) atomicOr(&bm[v >> 5], 1u << (v & 31));
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    return first_unselected(bm[lane]);
}

// ---------------------------------------- single-workgroup FPS: the list hit
//
// A run of list hits (see fps_single) as one hand-scheduled loop.  A wave on
// its own issues one instruction every four cycles, but a vector result read
// by the scalar unit (a compare's lane mask, a lane read feeding a scalar
// compare), a DPP operand written by the instruction just before it, and
// every branch each cost several issue slots when nothing independent sits
// in between.  The compiler's schedule leaves those gaps open at the end of
// the hit (lane maximum -> first lane -> winner's lane reads -> loop test);
// here the pulses' distance updates, cut into two-instruction parts, fill
// them.  Two hits per loop trip, the centroid alternating between two sets
// of scalar registers, one conditional branch per hit.  Arithmetic and
// operand order are those of sqd() and of the generic loop, so results are
// bit-identical.
//
// Per hit j (slot j, centroid c = set I):
//   selection s_j into lane j%64 of `sel` (lane select in m0);
//   the list entry's distance to c, its running minimum, the wave maximum wm
//   (six DPP steps, two independent instructions before each);
//   the winner: first lane with lv == wm, its five values into set O;
//   the pulses' update (distance, strict compare, slot and minimum selects);
//   j += 1; leave when wm <= U, or when j reaches jend (set by the caller at
//   the end of the 64-slot block of `sel`, or at P).
// Hazard rules kept: two VALU instructions between a VGPR write and a DPP read
// of it; at least one instruction between a VALU write of a scalar register
// (compare mask, lane read) and any read of it.

// one pulse's update in seven two-instruction parts; pulse k uses temporaries
// T0..T3, T alternating between e and a (the list's temporaries, free once
// the list distance is done); every pulse's compare mask goes to mk, read by
// its selects before the next pulse's compare writes it
#define FH_A(k, C, T) "v_subrev_f32 %[" #T "0], %[" #C "x], %[px" #k "]\n v_subrev_f32 %[" #T "1], %[" #C "y], %[py" #k "]\n"
#define FH_B(k, C, T) "v_subrev_f32 %[" #T "2], %[" #C "z], %[pz" #k "]\n v_subrev_f32 %[" #T "3], %[" #C "t], %[pt" #k "]\n"
#define FH_C(k, C, T) "v_mul_f32 %[" #T "0], %[" #T "0], %[" #T "0]\n v_mul_f32 %[" #T "1], %[" #T "1], %[" #T "1]\n"
#define FH_D(k, C, T) "v_mul_f32 %[" #T "2], %[" #T "2], %[" #T "2]\n v_mul_f32 %[" #T "3], %[" #T "3], %[" #T "3]\n"
#define FH_E(k, C, T) "v_add_f32 %[" #T "0], %[" #T "0], %[" #T "1]\n v_add_f32 %[" #T "0], %[" #T "0], %[" #T "2]\n"
#define FH_F(k, C, T) "v_add_f32 %[" #T "0], %[" #T "0], %[" #T "3]\n v_cmp_lt_f32_e64 %[mk], %[" #T "0], %[md" #k "]\n"
#define FH_G(k, C, T) "v_cndmask_b32_e64 %[nr" #k "], %[nr" #k "], %[vj], %[mk]\n v_cndmask_b32_e64 %[md" #k "], %[md" #k "], %[" #T "0], %[mk]\n"

// the list entry's distance and its running minimum
#define FH_LIST(C)                                                                       \
    "v_subrev_f32 %[a0], %[" #C "x], %[lx]\n v_subrev_f32 %[a1], %[" #C "y], %[ly]\n"    \
    "v_subrev_f32 %[a2], %[" #C "z], %[lz]\n v_subrev_f32 %[a3], %[" #C "t], %[lt]\n"    \
    "v_mul_f32 %[a0], %[a0], %[a0]\n v_mul_f32 %[a1], %[a1], %[a1]\n"                    \
    "v_mul_f32 %[a2], %[a2], %[a2]\n v_mul_f32 %[a3], %[a3], %[a3]\n"                    \
    "v_add_f32 %[a0], %[a0], %[a1]\n v_add_f32 %[a0], %[a0], %[a2]\n"                    \
    "v_add_f32 %[a0], %[a0], %[a3]\n v_min_i32 %[lv], %[a0], %[lv]\n"
#define FH_DPP1 "v_max_i32_dpp %[dd], %[dd], %[dd] quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
// the first step of a hit's reduction reads the list values themselves: a
// quad permute has a source in every lane, so every lane of dd is written
#define FH_DPP1L "v_max_i32_dpp %[dd], %[lv], %[lv] quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
#define FH_DPP2 "v_max_i32_dpp %[dd], %[dd], %[dd] quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n"
#define FH_DPP3 "v_max_i32_dpp %[dd], %[dd], %[dd] row_half_mirror row_mask:0xf bank_mask:0xf\n"
#define FH_DPP4 "v_max_i32_dpp %[dd], %[dd], %[dd] row_mirror row_mask:0xf bank_mask:0xf\n"
#define FH_DPP5 "v_max_i32_dpp %[dd], %[dd], %[dd] row_bcast:15 row_mask:0xa bank_mask:0xf\n"
#define FH_DPP6 "v_max_i32_dpp %[dd], %[dd], %[dd] row_bcast:31 row_mask:0xc bank_mask:0xf\n"
// the winner of the hit into set O; the slot counter and the exit bound
#define FH_WM "v_readlane_b32 %[wm], %[dd], 63\n"
#define FH_CMP "v_cmp_eq_u32_e64 %[mw], %[wm], %[lv]\n"
#define FH_FF1                                                                          \
    "s_ff1_i32_b64 %[lw], %[mw]\n s_add_u32 %[j], %[j], 1\n s_add_u32 m0, m0, 1\n"      \
    "s_cmp_eq_u32 %[j], %[jend]\n s_cselect_b32 %[ue], 0x7fffffff, %[U]\n"
#define FH_READ(O)                                                                      \
    "v_readlane_b32 %[" #O "x], %[lx], %[lw]\n v_readlane_b32 %[" #O "y], %[ly], %[lw]\n" \
    "v_readlane_b32 %[" #O "z], %[lz], %[lw]\n v_readlane_b32 %[" #O "t], %[lt], %[lw]\n" \
    "v_readlane_b32 %[" #O "s], %[li], %[lw]\n"
#define FH_HEAD(I) "v_writelane_b32 %[sel], %[" #I "s], m0\n v_mov_b32 %[vj], %[j]\n"

// One hit with the centroid in set I and the winner going to set O, for M
// pulses per lane.  P0..P20 are the pulses' parts in issue order.
#define FH_HIT(I, O, P0, P1, P2, P3, P4, P5, P6, P7, P8, P9, P10, TAIL)                     \
    FH_HEAD(I) FH_LIST(I) P0 FH_DPP1L P1 FH_DPP2 P2 FH_DPP3 P3 FH_DPP4 P4 FH_DPP5 P5 FH_DPP6  \
        P6 FH_WM P7 FH_CMP P8 P9 FH_FF1 P10 FH_READ(O) TAIL

// pulse part streams: pulse k's parts A..F, then the previous pulse's G one
// part later (so a compare's mask is never read by the next instruction)
#define FH_HIT1(I, O)                                                                        \
    FH_HIT(I, O, FH_A(0, I, e), FH_B(0, I, e), FH_C(0, I, e), FH_D(0, I, e), FH_E(0, I, e),  \
           FH_F(0, I, e), "s_nop 1\n", "s_nop 0\n", "s_nop 0\n", "", "", "s_nop 0\n" FH_G(0, I, e))
#define FH_HIT2(I, O)                                                                        \
    FH_HIT(I, O, FH_A(0, I, e), FH_B(0, I, e), FH_C(0, I, e), FH_D(0, I, e), FH_E(0, I, e),  \
           FH_F(0, I, e), FH_A(1, I, a), FH_G(0, I, e), FH_B(1, I, a), FH_C(1, I, a),       \
           FH_D(1, I, a), FH_E(1, I, a) FH_F(1, I, a) "s_nop 0\n" FH_G(1, I, a))
#define FH_HIT3(I, O)                                                                        \
    FH_HIT(I, O, FH_A(0, I, e), FH_B(0, I, e), FH_C(0, I, e), FH_D(0, I, e), FH_E(0, I, e),  \
           FH_F(0, I, e), FH_A(1, I, a), FH_G(0, I, e), FH_B(1, I, a), FH_C(1, I, a),       \
           FH_D(1, I, a),                                                                    \
           FH_E(1, I, a) FH_F(1, I, a) FH_A(2, I, e) FH_G(1, I, a) FH_B(2, I, e)             \
           FH_C(2, I, e) FH_D(2, I, e) FH_E(2, I, e) FH_F(2, I, e) "s_nop 0\n" FH_G(2, I, e))
// 4 to 8 pulses per lane: the same stream, the hits only (the exchange is
// the caller's)
#define FH_HIT4(I, O)                                                                         \
    FH_HIT(I, O, FH_A(0, I, e), FH_B(0, I, e), FH_C(0, I, e), FH_D(0, I, e), FH_E(0, I, e),    \
    FH_F(0, I, e), FH_A(1, I, a), FH_G(0, I, e), FH_B(1, I, a), FH_C(1, I, a), FH_D(1, I, a),  \
    FH_E(1, I, a) FH_F(1, I, a) FH_A(2, I, e) FH_G(1, I, a) FH_B(2, I, e) FH_C(2, I, e)        \
    FH_D(2, I, e) FH_E(2, I, e) FH_F(2, I, e) FH_A(3, I, a) FH_G(2, I, e) FH_B(3, I, a)        \
    FH_C(3, I, a) FH_D(3, I, a) FH_E(3, I, a) FH_F(3, I, a) "s_nop 0\n" FH_G(3, I, a))
#define FH_HIT5(I, O)                                                                         \
    FH_HIT(I, O, FH_A(0, I, e), FH_B(0, I, e), FH_C(0, I, e), FH_D(0, I, e), FH_E(0, I, e),    \
    FH_F(0, I, e), FH_A(1, I, a), FH_G(0, I, e), FH_B(1, I, a), FH_C(1, I, a), FH_D(1, I, a),  \
    FH_E(1, I, a) FH_F(1, I, a) FH_A(2, I, e) FH_G(1, I, a) FH_B(2, I, e) FH_C(2, I, e)        \
    FH_D(2, I, e) FH_E(2, I, e) FH_F(2, I, e) FH_A(3, I, a) FH_G(2, I, e) FH_B(3, I, a)        \
    FH_C(3, I, a) FH_D(3, I, a) FH_E(3, I, a) FH_F(3, I, a) FH_A(4, I, e) FH_G(3, I, a)        \
    FH_B(4, I, e) FH_C(4, I, e) FH_D(4, I, e) FH_E(4, I, e) FH_F(4, I, e) "s_nop 0\n"          \
    FH_G(4, I, e))
#define FH_HIT6(I, O)                                                                         \
    FH_HIT(I, O, FH_A(0, I, e), FH_B(0, I, e), FH_C(0, I, e), FH_D(0, I, e), FH_E(0, I, e),    \
    FH_F(0, I, e), FH_A(1, I, a), FH_G(0, I, e), FH_B(1, I, a), FH_C(1, I, a), FH_D(1, I, a),  \
    FH_E(1, I, a) FH_F(1, I, a) FH_A(2, I, e) FH_G(1, I, a) FH_B(2, I, e) FH_C(2, I, e)        \
    FH_D(2, I, e) FH_E(2, I, e) FH_F(2, I, e) FH_A(3, I, a) FH_G(2, I, e) FH_B(3, I, a)        \
    FH_C(3, I, a) FH_D(3, I, a) FH_E(3, I, a) FH_F(3, I, a) FH_A(4, I, e) FH_G(3, I, a)        \
    FH_B(4, I, e) FH_C(4, I, e) FH_D(4, I, e) FH_E(4, I, e) FH_F(4, I, e) FH_A(5, I, a)        \
    FH_G(4, I, e) FH_B(5, I, a) FH_C(5, I, a) FH_D(5, I, a) FH_E(5, I, a) FH_F(5, I, a)        \
    "s_nop 0\n" FH_G(5, I, a))
#define FH_HIT7(I, O)                                                                         \
    FH_HIT(I, O, FH_A(0, I, e), FH_B(0, I, e), FH_C(0, I, e), FH_D(0, I, e), FH_E(0, I, e),    \
    FH_F(0, I, e), FH_A(1, I, a), FH_G(0, I, e), FH_B(1, I, a), FH_C(1, I, a), FH_D(1, I, a),  \
    FH_E(1, I, a) FH_F(1, I, a) FH_A(2, I, e) FH_G(1, I, a) FH_B(2, I, e) FH_C(2, I, e)        \
    FH_D(2, I, e) FH_E(2, I, e) FH_F(2, I, e) FH_A(3, I, a) FH_G(2, I, e) FH_B(3, I, a)        \
    FH_C(3, I, a) FH_D(3, I, a) FH_E(3, I, a) FH_F(3, I, a) FH_A(4, I, e) FH_G(3, I, a)        \
    FH_B(4, I, e) FH_C(4, I, e) FH_D(4, I, e) FH_E(4, I, e) FH_F(4, I, e) FH_A(5, I, a)        \
    FH_G(4, I, e) FH_B(5, I, a) FH_C(5, I, a) FH_D(5, I, a) FH_E(5, I, a) FH_F(5, I, a)        \
    FH_A(6, I, e) FH_G(5, I, a) FH_B(6, I, e) FH_C(6, I, e) FH_D(6, I, e) FH_E(6, I, e)        \
    FH_F(6, I, e) "s_nop 0\n" FH_G(6, I, e))
#define FH_HIT8(I, O)                                                                         \
    FH_HIT(I, O, FH_A(0, I, e), FH_B(0, I, e), FH_C(0, I, e), FH_D(0, I, e), FH_E(0, I, e),    \
    FH_F(0, I, e), FH_A(1, I, a), FH_G(0, I, e), FH_B(1, I, a), FH_C(1, I, a), FH_D(1, I, a),  \
    FH_E(1, I, a) FH_F(1, I, a) FH_A(2, I, e) FH_G(1, I, a) FH_B(2, I, e) FH_C(2, I, e)        \
    FH_D(2, I, e) FH_E(2, I, e) FH_F(2, I, e) FH_A(3, I, a) FH_G(2, I, e) FH_B(3, I, a)        \
    FH_C(3, I, a) FH_D(3, I, a) FH_E(3, I, a) FH_F(3, I, a) FH_A(4, I, e) FH_G(3, I, a)        \
    FH_B(4, I, e) FH_C(4, I, e) FH_D(4, I, e) FH_E(4, I, e) FH_F(4, I, e) FH_A(5, I, a)        \
    FH_G(4, I, e) FH_B(5, I, a) FH_C(5, I, a) FH_D(5, I, a) FH_E(5, I, a) FH_F(5, I, a)        \
    FH_A(6, I, e) FH_G(5, I, a) FH_B(6, I, e) FH_C(6, I, e) FH_D(6, I, e) FH_E(6, I, e)        \
    FH_F(6, I, e) FH_A(7, I, a) FH_G(6, I, e) FH_B(7, I, a) FH_C(7, I, a) FH_D(7, I, a)        \
    FH_E(7, I, a) FH_F(7, I, a) "s_nop 0\n" FH_G(7, I, a))

// The exchange of the usual case, for 2 or 3 pulses per lane, in the same
// loop (label 5): the steps of the exchange in fps_single with the same
// LDS layout (SingleLds, parity ex & 1).  Each lane's farthest pulse and
// second distance; the wave's largest second distance by DPP; the offers
// (farthest >= that bound, and >= 0) written under an exec mask, their rank
// from mbcnt of exec; lane 0 writes the wave's count and bound; a barrier;
// every lane reads the four counts and bounds (U = the largest bound, >= 0);
// when the offers fit the list, lane l loads offer l of the waves'
// concatenation (lanes past the total: empty) and the list's maximum and
// first lane give the next centroid, into set 0; then the hits go on.
// Leaves the loop with code 1 (the list overflows: the caller's exchange
// redoes it with the next parity) or code 2 (every distance is 0: the list
// and U are new, the caller picks the lowest unselected pulse).
#define FH_BEST(k)                                                                         \
    "v_cmp_gt_i32_e64 %[mk], %[md" #k "], %[e0]\n v_max_i32 %[e3], %[e1], %[md" #k "]\n"      \
    "s_nop 0\n v_cndmask_b32_e64 %[e1], %[e3], %[e0], %[mk]\n"                              \
    "v_cndmask_b32_e64 %[e0], %[e0], %[md" #k "], %[mk]\n"                                  \
    "v_cndmask_b32_e64 %[e2], %[e2], " #k ", %[mk]\n"                                       \
    "v_cndmask_b32_e64 %[a0], %[a0], %[px" #k "], %[mk]\n"                                  \
    "v_cndmask_b32_e64 %[a1], %[a1], %[py" #k "], %[mk]\n"                                  \
    "v_cndmask_b32_e64 %[a2], %[a2], %[pz" #k "], %[mk]\n"                                  \
    "v_cndmask_b32_e64 %[a3], %[a3], %[pt" #k "], %[mk]\n"
#define FH_BEST0                                                                           \
    "v_mov_b32 %[e0], %[md0]\n v_bfrev_b32 %[e1], 1\n v_mov_b32 %[e2], 0\n"                 \
    "v_mov_b32 %[a0], %[px0]\n v_mov_b32 %[a1], %[py0]\n v_mov_b32 %[a2], %[pz0]\n"         \
    "v_mov_b32 %[a3], %[pt0]\n"
// The second centroid set (c1) is free during an exchange and serves as its
// scalar temporaries.  LDS layout the exchange addresses directly (SingleLds):
// ov at 0, oi at 2048, oc at 4096, wc at 12288, wb at 12320; parity p of
// ov/oi at +1024p, of oc at +4096p, of wc/wb at +16p; wave w at +256w
// (ov, oi), +1024w (oc), +4w (wc, wb).
#define FH_EXCH(BEST)                                                                      \
    "5:\n" FH_BEST0 BEST                                                                   \
    "v_mov_b32 %[dd], %[e1]\n v_add_u32 %[e2], %[e2], %[lb]\n s_nop 0\n"                    \
    FH_DPP1 "s_and_b32 %[c1y], %[ex], 1\n s_lshl_b32 %[c1y], %[c1y], 10\n"                   \
    FH_DPP2 "s_add_u32 %[c1y], %[c1y], %[lds]\n s_lshl_b32 %[ue], %[wave], 8\n"               \
    FH_DPP3 "s_add_u32 %[ue], %[ue], %[c1y]\n s_lshl_b32 %[lw], %[wave], 10\n"                \
    FH_DPP4 "s_add_u32 %[lw], %[lw], %[lds]\n s_add_u32 %[lw], %[lw], 0x1000\n"               \
    FH_DPP5 "s_and_b32 %[c1x], %[ex], 1\n s_lshl_b32 %[c1x], %[c1x], 12\n"                   \
    FH_DPP6 "s_add_u32 %[lw], %[lw], %[c1x]\n v_cmp_le_i32_e64 %[mw], 0, %[e0]\n"             \
    "v_readlane_b32 %[wm], %[dd], 63\n s_nop 0\n"                                          \
    "v_cmp_ge_i32_e64 %[mk], %[e0], %[wm]\n s_nop 0\n"                                      \
    "s_and_b64 %[mk], %[mk], %[mw]\n s_mov_b64 %[mw], exec\n s_mov_b64 exec, %[mk]\n"        \
    "s_nop 1\n"                                                                            \
    "v_mbcnt_lo_u32_b32 %[vj], exec_lo, 0\n v_mbcnt_hi_u32_b32 %[vj], exec_hi, %[vj]\n"     \
    "v_lshl_add_u32 %[dd], %[vj], 2, %[ue]\n v_lshl_add_u32 %[vj], %[vj], 4, %[lw]\n"        \
    "ds_write2st64_b32 %[dd], %[e0], %[e2] offset1:8\n"                                     \
    "ds_write2_b32 %[vj], %[a0], %[a1] offset1:1\n"                                         \
    "ds_write2_b32 %[vj], %[a2], %[a3] offset0:2 offset1:3\n"                               \
    "s_bcnt1_i32_b64 %[lw], %[mk]\n s_mov_b64 exec, 1\n"                                    \
    "s_and_b32 %[ue], %[ex], 1\n s_lshl_b32 %[ue], %[ue], 4\n s_add_u32 %[ue], %[ue], %[lds]\n" \
    "s_add_u32 %[ue], %[ue], 0x3000\n s_nop 0\n"                                            \
    "v_mov_b32 %[e1], %[lw]\n v_mov_b32 %[e3], %[wm]\n v_mov_b32 %[dd], %[wave]\n"          \
    "v_lshl_add_u32 %[dd], %[dd], 2, %[ue]\n"                                               \
    "ds_write2_b32 %[dd], %[e1], %[e3] offset1:8\n"                                         \
    "s_mov_b64 exec, %[mw]\n"                                                              \
    "s_waitcnt lgkmcnt(0)\n s_barrier\n"                                                   \
    "v_mov_b32 %[dd], %[ue]\n s_add_u32 %[c1x], %[c1x], %[lds]\n s_add_u32 %[c1x], %[c1x], 0x1000\n" \
    "ds_read_b32 %[e0], %[dd]\n ds_read_b32 %[e1], %[dd] offset:4\n"                        \
    "ds_read_b32 %[e2], %[dd] offset:8\n ds_read_b32 %[e3], %[dd] offset:12\n"              \
    "ds_read_b32 %[a0], %[dd] offset:32\n ds_read_b32 %[a1], %[dd] offset:36\n"             \
    "ds_read_b32 %[a2], %[dd] offset:40\n ds_read_b32 %[a3], %[dd] offset:44\n"             \
    "s_add_u32 %[ex], %[ex], 1\n"                                                          \
    "s_waitcnt lgkmcnt(0)\n"                                                               \
    "v_max3_i32 %[a0], %[a0], %[a1], %[a2]\n v_max3_i32 %[a0], %[a0], %[a3], 0\n"           \
    "v_add_u32 %[a1], %[e0], %[e1]\n v_add3_u32 %[a2], %[e0], %[e1], %[e2]\n"               \
    "v_add_u32 %[a3], %[a2], %[e3]\n"                                                      \
    "v_readfirstlane_b32 %[ue], %[a0]\n v_readfirstlane_b32 %[lw], %[a3]\n"                 \
    "v_cmp_ge_u32_e64 %[mk], %[lane], %[e0]\n v_mov_b32 %[dd], 0\n"                        \
    "v_cndmask_b32_e64 %[vj], 0, 1, %[mk]\n v_cndmask_b32_e64 %[dd], %[dd], %[e0], %[mk]\n" \
    "v_cmp_ge_u32_e64 %[mk], %[lane], %[a1]\n s_nop 0\n"                                   \
    "v_cndmask_b32_e64 %[vj], %[vj], 2, %[mk]\n v_cndmask_b32_e64 %[dd], %[dd], %[a1], %[mk]\n" \
    "v_cmp_ge_u32_e64 %[mk], %[lane], %[a2]\n s_nop 0\n"                                   \
    "v_cndmask_b32_e64 %[vj], %[vj], 3, %[mk]\n v_cndmask_b32_e64 %[dd], %[dd], %[a2], %[mk]\n" \
    "v_sub_u32 %[dd], %[lane], %[dd]\n"                                                    \
    "s_cmp_gt_i32 %[lw], 64\n s_cbranch_scc1 6f\n"                                          \
    "v_lshlrev_b32 %[e1], 8, %[vj]\n v_lshl_add_u32 %[e1], %[dd], 2, %[e1]\n"               \
    "v_add_u32 %[e1], %[c1y], %[e1]\n"                                                      \
    "v_lshlrev_b32 %[e2], 10, %[vj]\n v_lshl_add_u32 %[e2], %[dd], 4, %[e2]\n"              \
    "v_add_u32 %[e2], %[c1x], %[e2]\n"                                                      \
    "v_cmp_gt_u32_e64 %[mk], %[a3], %[lane]\n v_mov_b32 %[lv], 0xbf800000\n"               \
    "s_mov_b32 %[U], %[ue]\n s_mov_b64 %[mw], exec\n s_mov_b64 exec, %[mk]\n"               \
    "ds_read_b32 %[lv], %[e1]\n ds_read_b32 %[li], %[e1] offset:2048\n"                     \
    "ds_read_b32 %[lx], %[e2]\n ds_read_b32 %[ly], %[e2] offset:4\n"                        \
    "ds_read_b32 %[lz], %[e2] offset:8\n ds_read_b32 %[lt], %[e2] offset:12\n"              \
    "s_mov_b64 exec, %[mw]\n s_waitcnt lgkmcnt(0)\n"                                        \
    "s_nop 1\n" FH_DPP1L "s_nop 1\n" FH_DPP2 "s_nop 1\n" FH_DPP3 "s_nop 1\n" FH_DPP4 "s_nop 1\n"          \
    FH_DPP5 "s_nop 1\n" FH_DPP6 "s_nop 1\n"                                                 \
    "v_readlane_b32 %[wm], %[dd], 63\n s_nop 0\n"                                          \
    "v_cmp_eq_u32_e64 %[mk], %[wm], %[lv]\n"                                                \
    "s_cmp_lt_i32 %[wm], 1\n s_cbranch_scc1 7f\n"                                           \
    "s_ff1_i32_b64 %[lw], %[mk]\n s_nop 0\n"                                               \
    FH_READ(c0) "s_branch 1b\n"                                                            \
    "6:\n s_mov_b32 %[code], 1\n s_branch 4f\n"                                             \
    "7:\n s_mov_b32 %[code], 2\n s_branch 4f\n"

// the loop: two hits per trip; a hit whose list no longer decides goes to the
// exchange (or, for one pulse per lane, back to the caller); the last winner
// is left in set 0
#define FH_LOOP(HIT, EXCH)                                                                  \
    "s_mov_b32 %[m0s], m0\n s_and_b32 m0, %[j], 63\n s_mov_b32 %[code], 0\n"                 \
    "1:\n" HIT(c0, c1) "s_cmp_le_i32 %[wm], %[ue]\n s_cbranch_scc1 2f\n"                    \
    HIT(c1, c0) "s_cmp_le_i32 %[wm], %[ue]\n s_cbranch_scc0 1b\n"                           \
    "s_cmp_eq_u32 %[j], %[jend]\n s_cbranch_scc0 5f\n s_branch 4f\n"                        \
    "2:\n s_cmp_eq_u32 %[j], %[jend]\n s_cbranch_scc0 5f\n"                                 \
    "s_mov_b32 %[c0x], %[c1x]\n s_mov_b32 %[c0y], %[c1y]\n s_mov_b32 %[c0z], %[c1z]\n"        \
    " s_mov_b32 %[c0t], %[c1t]\n s_mov_b32 %[c0s], %[c1s]\n s_branch 4f\n"                   \
    EXCH                                                                                   \
    "4:\n s_mov_b32 m0, %[m0s]\n"
#define FH_EXCH1 "5:\n s_mov_b32 %[code], 1\n"

// the loop of hits only: leaves when a hit's list no longer decides or at
// jend; the last winner is left in set 0
#define FH_LOOPH(HIT)                                                                      \
    "s_mov_b32 %[m0s], m0\n s_and_b32 m0, %[j], 63\n s_nop 0\n"                            \
    "1:\n" HIT(c0, c1) "s_cmp_le_i32 %[wm], %[ue]\n s_cbranch_scc1 2f\n"                    \
    HIT(c1, c0) "s_cmp_le_i32 %[wm], %[ue]\n s_cbranch_scc0 1b\n s_branch 3f\n"              \
    "2:\n s_mov_b32 %[c0x], %[c1x]\n s_mov_b32 %[c0y], %[c1y]\n s_mov_b32 %[c0z], %[c1z]\n" \
    " s_mov_b32 %[c0t], %[c1t]\n s_mov_b32 %[c0s], %[c1s]\n"                               \
    "3:\n s_mov_b32 m0, %[m0s]\n"
#define FH_OUTSH                                                                             \
    [lv] "+v"(lvi), [sel] "+v"(sel), [c0x] "+s"(c0x), [c0y] "+s"(c0y), [c0z] "+s"(c0z),       \
        [c0t] "+s"(c0t), [c0s] "+s"(c0s), [c1x] "=&s"(c1x), [c1y] "=&s"(c1y),                 \
        [c1z] "=&s"(c1z), [c1t] "=&s"(c1t), [c1s] "=&s"(c1s), [j] "+s"(jj), [wm] "=&s"(wm),   \
        [ue] "=&s"(ue), [lw] "=&s"(lw), [mk] "=&s"(mk), [mw] "=&s"(mw), [a0] "=&v"(t0),       \
        [a1] "=&v"(t1), [a2] "=&v"(t2), [a3] "=&v"(t3), [e0] "=&v"(t4), [e1] "=&v"(t5),       \
        [e2] "=&v"(t6), [e3] "=&v"(t7), [dd] "=&v"(t8), [vj] "=&v"(t9), [m0s] "=&s"(m0s)
#define FH_INSH                                                                              \
    [lx] "v"(lx), [ly] "v"(ly), [lz] "v"(lz), [lt] "v"(lt), [li] "v"(li), [U] "s"(U),         \
        [jend] "s"(jend)

#define FH_PULSE_IO(k) [md##k] "+v"(md[k]), [nr##k] "+v"(nr[k])
#define FH_PULSE_IN(k) [px##k] "v"(px[k]), [py##k] "v"(py[k]), [pz##k] "v"(pz[k]), [pt##k] "v"(pt[k])
#define FH_OUTS                                                                              \
    [lv] "+v"(lvi), [sel] "+v"(sel), [lx] "+v"(lx), [ly] "+v"(ly), [lz] "+v"(lz),             \
        [lt] "+v"(lt), [li] "+v"(li), [U] "+s"(U), [ex] "+s"(ex), [code] "=&s"(code),          \
        [c0x] "+s"(c0x), [c0y] "+s"(c0y), [c0z] "+s"(c0z),       \
        [c0t] "+s"(c0t), [c0s] "+s"(c0s), [c1x] "=&s"(c1x), [c1y] "=&s"(c1y),                 \
        [c1z] "=&s"(c1z), [c1t] "=&s"(c1t), [c1s] "=&s"(c1s), [j] "+s"(jj), [wm] "=&s"(wm),   \
        [ue] "=&s"(ue), [lw] "=&s"(lw), [mk] "=&s"(mk), [mw] "=&s"(mw),                      \
        [a0] "=&v"(t0), [a1] "=&v"(t1), [a2] "=&v"(t2), [a3] "=&v"(t3),       \
        [e0] "=&v"(t4), [e1] "=&v"(t5), [e2] "=&v"(t6), [e3] "=&v"(t7), [dd] "=&v"(t8),       \
        [vj] "=&v"(t9), [m0s] "=&s"(m0s)
#define FH_INS                                                                               \
    [jend] "s"(jend), [lds] "s"(lds), [wave] "s"(wave), [lane] "v"(lane), [lb] "v"(lbase)

// Runs list hits from slot j, with the exchanges of the usual case in
// between, until j + 1 reaches jend (the end of the 64-slot block of `sel`,
// or P; code 0), an exchange overflows the list (code 1: the caller's
// exchange redoes it) or finds every distance 0 (code 2: the list and U are
// new, the caller picks the lowest unselected pulse).  Returns with j = the
// last slot done, wm its list maximum, (s, c) the winner of that hit, and
// the list, U and the exchange count ex as they stand.  sel collects the
// selections of the block (lane q: slot 64*(j/64) + q).
template <int M>
__device__ __forceinline__ int fps_hit_run(const float (&px)[M], const float (&py)[M],
                                           const float (&pz)[M], const float (&pt)[M],
                                           float (&md)[M], int (&nr)[M], float& lv, float& lx,
                                           float& ly, float& lz, float& lt, int& li, int& U,
                                           int& ex, int jend, int& j, int& wm_out, int& s,
                                           float& cx, float& cy, float& cz, float& ct, int& sel,
                                           SingleLds& L, int wave, int lane, int lbase) {
    // every scalar operand is uniform; readfirstlane says so to the compiler
    const auto u = [](float v) {
        return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
    };
    int lvi = __float_as_int(lv);
    float c0x = u(cx), c0y = u(cy), c0z = u(cz), c0t = u(ct), c1x, c1y, c1z, c1t;
    int c0s = __builtin_amdgcn_readfirstlane(s), c1s, wm, ue, lw, code;
    int jj = __builtin_amdgcn_readfirstlane(j);
    U = __builtin_amdgcn_readfirstlane(U);
    ex = __builtin_amdgcn_readfirstlane(ex);
    jend = __builtin_amdgcn_readfirstlane(jend);
    wave = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(&L));
    uint64_t mk, mw;
    float t0, t1, t2, t3, t4, t5, t6, t7, t8, t9;  // temporaries
    int m0s;  // m0 (the lane select of v_writelane) is saved and restored
    if constexpr (M == 1) {
        asm volatile(FH_LOOP(FH_HIT1, FH_EXCH1) : FH_PULSE_IO(0), FH_OUTS : FH_PULSE_IN(0), FH_INS
                     : "scc", "memory");
    } else if constexpr (M == 2) {
        asm volatile(FH_LOOP(FH_HIT2, FH_EXCH(FH_BEST(1)))
                     : FH_PULSE_IO(0), FH_PULSE_IO(1), FH_OUTS
                     : FH_PULSE_IN(0), FH_PULSE_IN(1), FH_INS : "scc", "memory");
    } else {
        static_assert(M == 3, "hand-scheduled hits for 1 to 3 pulses per lane");
        asm volatile(FH_LOOP(FH_HIT3, FH_EXCH(FH_BEST(1) FH_BEST(2)))
                     : FH_PULSE_IO(0), FH_PULSE_IO(1), FH_PULSE_IO(2), FH_OUTS
                     : FH_PULSE_IN(0), FH_PULSE_IN(1), FH_PULSE_IN(2), FH_INS : "scc", "memory");
    }
    lv = __int_as_float(lvi);
    j = jj - 1;
    wm_out = wm;
    s = c0s;
    cx = c0x;
    cy = c0y;
    cz = c0z;
    ct = c0t;
    return code;
}

// Runs list hits only (4 to 8 pulses per lane) from slot j until a hit's
// list no longer decides (wm <= U) or j + 1 reaches jend; returns with j =
// the last slot done, wm its list maximum and (s, c) the winner of that hit.
template <int M>
__device__ __forceinline__ void fps_hit_run_h(const float (&px)[M], const float (&py)[M],
                                              const float (&pz)[M], const float (&pt)[M],
                                              float (&md)[M], int (&nr)[M], float& lv, float lx,
                                              float ly, float lz, float lt, int li, int U,
                                              int jend, int& j, int& wm_out, int& s, float& cx,
                                              float& cy, float& cz, float& ct, int& sel) {
    const auto u = [](float v) {
        return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
    };
    int lvi = __float_as_int(lv);
    float c0x = u(cx), c0y = u(cy), c0z = u(cz), c0t = u(ct), c1x, c1y, c1z, c1t;
    int c0s = __builtin_amdgcn_readfirstlane(s), c1s, wm, ue, lw;
    int jj = __builtin_amdgcn_readfirstlane(j);
    U = __builtin_amdgcn_readfirstlane(U);
    jend = __builtin_amdgcn_readfirstlane(jend);
    uint64_t mk, mw;
    float t0, t1, t2, t3, t4, t5, t6, t7, t8, t9;  // temporaries
    int m0s;
#define FH_IO4 FH_PULSE_IO(0), FH_PULSE_IO(1), FH_PULSE_IO(2), FH_PULSE_IO(3)
#define FH_IN4 FH_PULSE_IN(0), FH_PULSE_IN(1), FH_PULSE_IN(2), FH_PULSE_IN(3)
    if constexpr (M == 4) {
        asm volatile(FH_LOOPH(FH_HIT4) : FH_IO4, FH_OUTSH : FH_IN4, FH_INSH : "scc");
    } else if constexpr (M == 5) {
        asm volatile(FH_LOOPH(FH_HIT5) : FH_IO4, FH_PULSE_IO(4), FH_OUTSH
                     : FH_IN4, FH_PULSE_IN(4), FH_INSH : "scc");
    } else if constexpr (M == 6) {
        asm volatile(FH_LOOPH(FH_HIT6) : FH_IO4, FH_PULSE_IO(4), FH_PULSE_IO(5), FH_OUTSH
                     : FH_IN4, FH_PULSE_IN(4), FH_PULSE_IN(5), FH_INSH : "scc");
    } else if constexpr (M == 7) {
        asm volatile(FH_LOOPH(FH_HIT7)
                     : FH_IO4, FH_PULSE_IO(4), FH_PULSE_IO(5), FH_PULSE_IO(6), FH_OUTSH
                     : FH_IN4, FH_PULSE_IN(4), FH_PULSE_IN(5), FH_PULSE_IN(6), FH_INSH : "scc");
    } else {
        static_assert(M == 8, "hand-scheduled hits only for 4 to 8 pulses per lane");
        asm volatile(FH_LOOPH(FH_HIT8)
                     : FH_IO4, FH_PULSE_IO(4), FH_PULSE_IO(5), FH_PULSE_IO(6), FH_PULSE_IO(7),
                       FH_OUTSH
                     : FH_IN4, FH_PULSE_IN(4), FH_PULSE_IN(5), FH_PULSE_IN(6), FH_PULSE_IN(7),
                       FH_INSH
                     : "scc");
    }
#undef FH_IO4
#undef FH_IN4
    lv = __int_as_float(lvi);
    j = jj - 1;
    wm_out = wm;
    s = c0s;
    cx = c0x;
    cy = c0y;
    cz = c0z;
    ct = c0t;
}

// FPS of one event of at most 256*M pulses by one workgroup, every pulse in
// registers (lane-blocked: thread t owns pulses t*M .. t*M+M-1).
//
// The argmax is exact but is computed from a cached candidate list most of
// the time.  Minimum distances only decrease, so if at some iteration every
// pulse outside a list has min distance <= U, that stays true afterwards;
// while the best listed pulse (its min distance kept current alongside the
// pulses) is > U it is the farthest pulse, ties included: every pulse with
// that distance is listed and the list is in pulse order.
//
// When the test fails (and at the first iteration) the workgroup exchanges:
//  * every group of pulses -- a lane's M pulses, or a pair of lanes when
//    M = 1 -- offers its farthest pulse (lowest index on ties), and its
//    second largest distance bounds the rest of the group;
//  * a wave keeps the offers >= the largest second distance of the wave
//    (padding never offers) and writes them, in lane order, to LDS with
//    their count; U is the largest wave bound;
//  * after a barrier every wave reads the counts and bounds; when all the
//    offers fit the list (the usual case) lane l reads offer l of the
//    waves' concatenation, which is in pulse order, and that is the new
//    list: it holds every pulse > U (such a pulse is the unique farthest of
//    its group and beats its wave's bound), offers <= U in it never win
//    while the list beats U, and its best entry is this iteration's argmax
//    (the global maximum is offered, and the lowest index among equal
//    maxima is the farthest of the lowest group holding one).  Otherwise
//    the offers > U become the list in pulse order through a second
//    barrier; beyond 64 the first 64 are kept and U is raised to the
//    largest of the others.
// Every wave holds the same list (lane l: entry l) and takes the same
// decisions; between exchanges the waves never synchronise.  One wave on a
// SIMD issues a vector instruction only every few cycles, so a run of list
// hits is kept to one short straight loop: the list's distances and their
// wave maximum, the pulses' update, a ballot and five lane reads for the
// winner; the centroid stays in scalar registers.  U is kept >= 0, so a
// maximum of 0 (every pulse selected or duplicate) always goes through an
// exchange, where the "lowest unselected index" rule is applied.  Every
// wave writes iteration j's selection to s_sel[j] (the same value from
// all: one LDS store, no branch).
template <int M>
__device__ __forceinline__ void fps_single(const SampleArgs& a, int64_t b, int64_t off, int n,
                                           int s0, SingleLds& L, int* s_sel, int* s_asg,
                                           const Stage& st) {
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int P = a.P;
    const float4* __restrict__ p = a.coords + off;
    const int lbase = tid * M;

    float px[M], py[M], pz[M], pt[M], md[M];
    int nr[M];
#pragma unroll
    for (int k = 0; k < M; ++k) {
        const int i = lbase + k;
        float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < n) q = p[i];
        px[k] = q.x;
        py[k] = q.y;
        pz[k] = q.z;
        pt[k] = q.w;
        md[k] = i < n ? INFINITY : -1.0f;  // padding never wins and is never updated
        nr[k] = 0;
    }
    // candidate list entry of this lane (-1: none)
    float lv = -1.0f, lx = 0.f, ly = 0.f, lz = 0.f, lt = 0.f;
    int li = 0;
    int U = INT32_MAX;  // bound on every unlisted pulse (float bits); no list yet
    int ex = 0;         // exchanges so far (their parity picks the offer buffer)

    int s = s0;
    float cx, cy, cz, ct;  // the newest centroid (uniform)
    {
        const float4 q = p[s];
        cx = readlane_f(q.x, 0);
        cy = readlane_f(q.y, 0);
        cz = readlane_f(q.z, 0);
        ct = readlane_f(q.w, 0);
    }
    float fr[kStageR];
    const int sr = __builtin_amdgcn_readfirstlane((st.nf + kFpsT - 1) / kFpsT);
#pragma unroll
    for (int r = 0; r < kStageR; ++r)
        if (r < sr) fr[r] = st.src[min(tid + kFpsT * r, st.nf - 1)];
    int j = 0;
    for (;;) {
        // ---- a run of iterations decided by the list
        int wm;
        if constexpr (M <= 3) {
            const int j0 = j;
            const int jb = j & ~63;
            int sel = 0;
            const int code = fps_hit_run<M>(px, py, pz, pt, md, nr, lv, lx, ly, lz, lt, li, U, ex,
                                            min(P, jb + 64), j, wm, s, cx, cy, cz, ct, sel, L,
                                            wave, lane, lbase);
            // the selections of slots j0..j (one 64-slot block)
            if (lane >= (j0 & 63) && lane <= (j & 63)) s_sel[jb + lane] = sel;
            if (code == 2) {
                // the exchange found every distance 0: the lowest unselected pulse
                s = min(first_unselected_sel(L.bm[wave], s_sel, j), n - 1);
                const float4 q = p[s];
                cx = readlane_f(q.x, 0);
                cy = readlane_f(q.y, 0);
                cz = readlane_f(q.z, 0);
                ct = readlane_f(q.w, 0);
                ++j;
                continue;
            }
            if (code == 1) wm = INT32_MIN;  // the exchange below redoes it
        } else if constexpr (M <= 8) {
            const int j0 = j;
            const int jb = j & ~63;
            int sel = 0;
            fps_hit_run_h<M>(px, py, pz, pt, md, nr, lv, lx, ly, lz, lt, li, U, min(P, jb + 64), j,
                             wm, s, cx, cy, cz, ct, sel);
            if (lane >= (j0 & 63) && lane <= (j & 63)) s_sel[jb + lane] = sel;
        } else for (;;) {
            s_sel[j] = s;
            // distances are >= +0, so their bit patterns order as signed
            // integers, and an empty entry (-1.0, negative) stays empty
            lv = __int_as_float(min(__float_as_int(sqd(lx, ly, lz, lt, cx, cy, cz, ct)),
                                    __float_as_int(lv)));
            wm = wave_max_i(__float_as_int(lv));
#pragma unroll
            for (int k = 0; k < M; ++k) {
                const float d = sqd(px[k], py[k], pz[k], pt[k], cx, cy, cz, ct);
                const bool u = d < md[k];
                nr[k] = u ? j : nr[k];
                md[k] = u ? d : md[k];
            }
            // the best listed pulse (lanes hold the list in pulse order),
            // read before the test: when the run ends here the exchange
            // replaces it
            const int Lw = (int)__builtin_ctzll(ballot(__float_as_int(lv) == wm));
            s = readlane_i(li, Lw);
            cx = readlane_f(lx, Lw);
            cy = readlane_f(ly, Lw);
            cz = readlane_f(lz, Lw);
            ct = readlane_f(lt, Lw);
            if (__builtin_expect(wm <= U, 0)) break;
            if (__builtin_expect(j + 1 == P, 0)) break;
            ++j;
        }
        if (j + 1 == P) break;
        if constexpr (M <= 8) {
            if (wm > U) {
                // the run stopped at the end of a block of selections: the
                // list still decides the next slot
                ++j;
                continue;
            }
        }

        // ---- exchange
        const int par = ex & 1;
        ++ex;
        int b1 = INT32_MIN, b2 = INT32_MIN, k1 = 0;
        float bx = 0.f, by = 0.f, bz = 0.f, bt = 0.f;
#pragma unroll
        for (int k = 0; k < M; ++k) {
            const int v = __float_as_int(md[k]);
            const bool g = v > b1;
            b2 = g ? b1 : max(b2, v);
            b1 = g ? v : b1;
            k1 = g ? k : k1;
            bx = g ? px[k] : bx;
            by = g ? py[k] : by;
            bz = g ? pz[k] : bz;
            bt = g ? pt[k] : bt;
        }
        bool lead = true;
        if (M == 1) {
            // groups are lane pairs (2l, 2l+1)
            const int q = dpp_i<kQuadSwap1, 0xF>(b1, INT32_MIN);
            lead = b1 > q || (b1 == q && (lane & 1) == 0);
            b2 = min(b1, q);
        }
        const int wb2 = wave_max_i(b2);
        const bool offer = lead && b1 >= wb2 && b1 >= 0;
        const uint64_t ob = ballot(offer);
        if (offer) {
            const int q = mbcnt(ob);
            L.ov[par][wave][q] = b1;
            L.oi[par][wave][q] = lbase + k1;
            L.oc[par][wave][q] = make_float4(bx, by, bz, bt);
        }
        if (lane == 0) {
            reinterpret_cast<int*>(&L.wc[par])[wave] = __popcll(ob);
            reinterpret_cast<int*>(&L.wb[par])[wave] = wb2;
        }
        lds_barrier();
        int cw[kFpsW], Un = 0, tot = 0;
        {
            const int4 c4 = L.wc[par];
            const int4 b4 = L.wb[par];
            cw[0] = __builtin_amdgcn_readfirstlane(c4.x);
            cw[1] = __builtin_amdgcn_readfirstlane(c4.y);
            cw[2] = __builtin_amdgcn_readfirstlane(c4.z);
            cw[3] = __builtin_amdgcn_readfirstlane(c4.w);
            Un = max(max(Un, (int)__builtin_amdgcn_readfirstlane(b4.x)),
                     max((int)__builtin_amdgcn_readfirstlane(b4.y),
                         max((int)__builtin_amdgcn_readfirstlane(b4.z),
                             (int)__builtin_amdgcn_readfirstlane(b4.w))));
            tot = cw[0] + cw[1] + cw[2] + cw[3];
        }
        int gm;
        if (__builtin_expect(tot <= kListCap, 1)) {
            // the new list: lane l holds offer l of the concatenation
            int w = 0, q = lane;
#pragma unroll
            for (int r = 0; r < kFpsW - 1; ++r) {
                const bool on = w == r && q >= cw[r];
                q = on ? q - cw[r] : q;
                w = on ? r + 1 : w;
            }
            if (lane < tot) {
                lv = __int_as_float(L.ov[par][w][q]);
                li = L.oi[par][w][q];
                const float4 c = L.oc[par][w][q];
                lx = c.x;
                ly = c.y;
                lz = c.z;
                lt = c.w;
            } else {
                lv = -1.0f;
            }
            U = __builtin_amdgcn_readfirstlane(Un);
            gm = wave_max_i(__float_as_int(lv));
            if (gm > 0) {
                const int Lw = (int)__builtin_ctzll(ballot(__float_as_int(lv) == gm));
                s = readlane_i(li, Lw);
                cx = readlane_f(lx, Lw);
                cy = readlane_f(ly, Lw);
                cz = readlane_f(lz, Lw);
                ct = readlane_f(lt, Lw);
            }
        } else {
            // every wave: this iteration's argmax (largest offer, then lowest
            // (wave, position) = lowest pulse index) and the list layout
            int rb = INT32_MIN, re = 0;
            int kcnt[kFpsW];
#pragma unroll
            for (int w = 0; w < kFpsW; ++w) {
                const int v = lane < cw[w] ? L.ov[par][w][lane] : INT32_MIN;
                const bool g = v > rb;
                rb = g ? v : rb;
                re = g ? w : re;
                kcnt[w] = __popcll(ballot(v > Un));
            }
            gm = wave_max_i(rb);
            if (gm > 0) {
                const uint64_t m = ballot(rb == gm);
                int Lw, ew;
                if (__popcll(m) == 1) {
                    Lw = (int)__builtin_ctzll(m);
                    ew = readlane_i(re, Lw);
                } else {
                    const int f = wave_min_i(rb == gm ? re * 64 + lane : INT32_MAX);
                    Lw = f & 63;
                    ew = f >> 6;
                }
                s = min(max((int)__builtin_amdgcn_readfirstlane(L.oi[par][ew][Lw]), 0), n - 1);
                const float4 c = L.oc[par][ew][Lw];
                cx = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(c.x)));
                cy = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(c.y)));
                cz = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(c.z)));
                ct = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(c.w)));
            }
            // new list: the offers > U in (wave, position) order, each wave
            // writing its own from registers; beyond 64 entries the rest only
            // raise U
            int base = 0, C = 0;
#pragma unroll
            for (int w = 0; w < kFpsW; ++w) {
                base += w < wave ? kcnt[w] : 0;
                C += kcnt[w];
            }
            const bool keep = offer && b1 > Un;
            const int pos = base + mbcnt(ballot(keep));
            if (keep && pos < kListCap) {
                FpsSlot& o = L.list[pos];
                o.v = __int_as_float(b1);
                o.i = lbase + k1;
                o.c = make_float4(bx, by, bz, bt);
            }
            if (C > kListCap) {
                const int d = wave_max_i(keep && pos >= kListCap ? b1 : INT32_MIN);
                // every wave needs the same U: combine the per-wave maxima
                if (lane == 0) L.wd[wave] = d;
                lds_barrier();
#pragma unroll
                for (int w = 0; w < kFpsW; ++w)
                    Un = max(Un, (int)__builtin_amdgcn_readfirstlane(L.wd[w]));
            }
            lds_barrier();
            U = __builtin_amdgcn_readfirstlane(Un);
            if (lane < C) {
                const FpsSlot o = L.list[lane];
                lv = o.v;
                li = o.i;
                lx = o.c.x;
                ly = o.c.y;
                lz = o.c.z;
                lt = o.c.w;
            } else {
                lv = -1.0f;
            }
        }
        if (gm <= 0) {
            // every pulse has minimum distance 0: the lowest unselected index
            s = min(first_unselected_sel(L.bm[wave], s_sel, j), n - 1);
            const float4 q = p[s];
            cx = readlane_f(q.x, 0);
            cy = readlane_f(q.y, 0);
            cz = readlane_f(q.z, 0);
            ct = readlane_f(q.w, 0);
        }
        ++j;
    }
    if (a.assign) {
#pragma unroll
        for (int k = 0; k < M; ++k) {
            const int i = lbase + k;
            if (i < n) a.assign[off + i] = nr[k];
        }
    }
    if (s_asg) {
        // every lane's M entries (below 256 * M <= kFpsCap); the sort reads
        // the first n
#pragma unroll
        for (int k = 0; k < M; ++k) s_asg[lbase + k] = nr[k];
    }
    // the rows and the zero row, with no per-lane branches: a row r is
    // written whole (uniform test) and its lanes beyond the rows store 0
    // (they stay below kStage, inside dst)
    const int sz = __builtin_amdgcn_readfirstlane((st.nz + kFpsT - 1) / kFpsT);
#pragma unroll
    for (int r = 0; r < kStageR; ++r) {
        if (r < sz) {
            const int q = tid + kFpsT * r;
            st.dst[q] = q < st.nf ? fr[r] : 0.0f;
        }
    }
    if (!st.defer_sel) write_selection(a, b, p, s_sel);
}

__device__ __forceinline__ void fps_single_dispatch(const SampleArgs& a, int64_t b, int64_t off,
                                                    int n, int s0, SingleLds& L, int* ss, int* sa,
                                                    const Stage& st) {
    switch ((n + kFpsT - 1) / kFpsT) {
        case 1: fps_single<1>(a, b, off, n, s0, L, ss, sa, st); break;
        case 2: fps_single<2>(a, b, off, n, s0, L, ss, sa, st); break;
        case 3: fps_single<3>(a, b, off, n, s0, L, ss, sa, st); break;
        case 4: fps_single<4>(a, b, off, n, s0, L, ss, sa, st); break;
        case 5: fps_single<5>(a, b, off, n, s0, L, ss, sa, st); break;
        case 6: fps_single<6>(a, b, off, n, s0, L, ss, sa, st); break;
        case 7: fps_single<7>(a, b, off, n, s0, L, ss, sa, st); break;
        case 8: fps_single<8>(a, b, off, n, s0, L, ss, sa, st); break;
        case 9: case 10: fps_single<10>(a, b, off, n, s0, L, ss, sa, st); break;
        case 11: case 12: fps_single<12>(a, b, off, n, s0, L, ss, sa, st); break;
        case 13: case 14: fps_single<14>(a, b, off, n, s0, L, ss, sa, st); break;
        default: fps_single<16>(a, b, off, n, s0, L, ss, sa, st); break;
    }
}

// ----------------------------------------- gang FPS, shared candidate list

constexpr int kGangE = 4;                 // gang-list entries per lane
constexpr int kGangCap = 64 * kGangE;     // entries of the gang list
constexpr int kRecSlots = 64;             // entries a shard publishes per exchange
constexpr int kRecBound = kRecSlots;      // record word holding the shard's bound
constexpr int kGangQ = kGangMax * kRecSlots / kFpsT;  // record entries read per thread at most

struct GangLds {
    FpsLds w;                   // the workgroup's own exchange
    FpsSlot glist[kGangCap];    // the new gang list
    FpsSlot gwin;               // the gang's argmax of an exchange
    int gU;                     // the gang's bound
    int gcnt[kGangQ * kFpsW];   // kept record entries per (read round, wave)
    int gdrop[kFpsW];
};

// A record word: tag (14 bits: the iteration + 1, at most 1025) | pulse
// index (18 bits, < kGangMax * kFpsCap) | distance bits (32).  One word per
// entry, so one relaxed agent-scope load sees a whole entry; the
// coordinates are read back from the (read-only) input.
__device__ __forceinline__ unsigned long long rec_word(int tag, int idx, int v) {
    return ((unsigned long long)(uint32_t)tag << 50) |
           ((unsigned long long)((uint32_t)idx & 0x3FFFFu) << 32) | (uint32_t)v;
}
__device__ __forceinline__ unsigned long long rec_load(const unsigned long long* w) {
    return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void rec_store(unsigned long long* w, unsigned long long word) {
    __hip_atomic_store(w, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool rec_ok(unsigned long long w, int tag) {
    return (uint32_t)(w >> 50) == (uint32_t)tag;
}
__device__ __forceinline__ int rec_idx(unsigned long long w) { return (int)((w >> 32) & 0x3FFFFu); }
__device__ __forceinline__ int rec_val(unsigned long long w) { return (int)(uint32_t)w; }

// FPS over one shard of an event shared by a gang of G workgroups (shard g
// holds pulses lo .. lo+cnt-1, at most 256*M, in registers as in
// fps_single).  The same exact candidate-list scheme, one level up: every
// shard holds the same gang-wide list (up to 256 entries, entry f = 64*e +
// lane in register e) and decides alone while the best listed pulse beats
// the gang bound U.  An exchange (the first iteration, and whenever the test
// fails):
//  1. inside the workgroup, as in fps_single: offers, the shard's best
//     pulse, its bound U_g and its offers > U_g (the first 63 in pulse
//     order; any others raise U_g);
//  2. the shard publishes a record: those entries in slots 0..62, its best
//     pulse in slot 63 and U_g, one 64-bit word each, tagged with the
//     iteration so that no ordering between the words is needed (relaxed
//     agent-scope atomics; records are double-buffered by exchange parity);
//  3. every workgroup polls all G records (bounded waits), takes the best of
//     the G shard bests (lowest shard on ties: lowest pulse index) as this
//     iteration's argmax, U = max U_g, and the record entries > U, in
//     (shard, slot) order, as the new gang list (the first 256; any others
//     raise U).  A shard's best may also sit among its slots 0..62; the
//     copy is harmless, and on ties the lowest (shard, slot) is still the
//     lowest pulse index.
// Returns the number of exchanges (the parity of the record buffer that no
// shard reads any more).
template <int M>
__device__ __forceinline__ int fps_gang(const SampleArgs& a, int64_t b, int64_t off, int n, int s0,
                                        const Shard& sh, GangLds& L, int* s_sel, int* s_asg) {
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int P = a.P;
    const int G = sh.G;
    const float4* __restrict__ p = a.coords + off;
    const int lbase = sh.lo + tid * M;  // event-local index of this lane's first pulse
    const int send = sh.lo + sh.cnt;
    __builtin_amdgcn_s_setprio(2);

    float px[M], py[M], pz[M], pt[M], md[M];
    int nr[M];
#pragma unroll
    for (int k = 0; k < M; ++k) {
        const int i = lbase + k;
        float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < send) q = p[i];
        px[k] = q.x;
        py[k] = q.y;
        pz[k] = q.z;
        pt[k] = q.w;
        md[k] = i < send ? INFINITY : -1.0f;
        nr[k] = 0;
    }
    float lv[kGangE], lx[kGangE], ly[kGangE], lz[kGangE], lt[kGangE];
    int li[kGangE];
#pragma unroll
    for (int e = 0; e < kGangE; ++e) {
        lv[e] = -1.0f;
        li[e] = 0;
        lx[e] = ly[e] = lz[e] = lt[e] = 0.f;
    }
    int nreg = 0;
    int U = INT32_MAX;
    int ex = 0;

    int selv = 0;
    int s = s0;
    float cx, cy, cz, ct;
    {
        const float4 q = p[s];
        cx = readlane_f(q.x, 0);
        cy = readlane_f(q.y, 0);
        cz = readlane_f(q.z, 0);
        ct = readlane_f(q.w, 0);
    }
    int j = 0;
    for (;;) {
        for (;;) {
            selv = lane == (j & 63) ? s : selv;
            if (__builtin_expect((j & 63) == 63 && wave == 0, 0)) s_sel[j - 63 + lane] = selv;
            int lb = INT32_MIN, le = 0;
#pragma unroll
            for (int e = 0; e < kGangE; ++e) {
                if (e < nreg) {
                    const float d = sqd(lx[e], ly[e], lz[e], lt[e], cx, cy, cz, ct);
                    lv[e] = d < lv[e] ? d : lv[e];
                    const int v = __float_as_int(lv[e]);
                    const bool g = v > lb;
                    lb = g ? v : lb;
                    le = g ? e : le;
                }
            }
            const int wm = wave_max_i(lb);
#pragma unroll
            for (int k = 0; k < M; ++k) {
                const float d = sqd(px[k], py[k], pz[k], pt[k], cx, cy, cz, ct);
                const bool u = d < md[k];
                nr[k] = u ? j : nr[k];
                md[k] = u ? d : md[k];
            }
            if (__builtin_expect(j + 1 == P || wm <= U, 0)) break;
            const uint64_t m = ballot(lb == wm);
            int Lw, ew;
            if (__popcll(m) == 1) {
                Lw = (int)__builtin_ctzll(m);
                ew = readlane_i(le, Lw);
            } else {
                const int f = wave_min_i(lb == wm ? le * 64 + lane : INT32_MAX);
                Lw = f & 63;
                ew = f >> 6;
            }
            int oi = li[0];
            float ox = lx[0], oy = ly[0], oz = lz[0], ot = lt[0];
#pragma unroll
            for (int e = 1; e < kGangE; ++e) {
                const bool t = ew == e;
                oi = t ? li[e] : oi;
                ox = t ? lx[e] : ox;
                oy = t ? ly[e] : oy;
                oz = t ? lz[e] : oz;
                ot = t ? lt[e] : ot;
            }
            s = readlane_i(oi, Lw);
            cx = readlane_f(ox, Lw);
            cy = readlane_f(oy, Lw);
            cz = readlane_f(oz, Lw);
            ct = readlane_f(ot, Lw);
            ++j;
        }
        if (j + 1 == P) break;

        // ---- 1. the workgroup's offers, best pulse, bound and entries
        int b1 = INT32_MIN, b2 = INT32_MIN, k1 = 0;
        float bx = 0.f, by = 0.f, bz = 0.f, bt = 0.f;
#pragma unroll
        for (int k = 0; k < M; ++k) {
            const int v = __float_as_int(md[k]);
            const bool g = v > b1;
            b2 = g ? b1 : max(b2, v);
            b1 = g ? v : b1;
            k1 = g ? k : k1;
            bx = g ? px[k] : bx;
            by = g ? py[k] : by;
            bz = g ? pz[k] : bz;
            bt = g ? pt[k] : bt;
        }
        const int wb2 = wave_max_i(b2);
        const bool offer = b1 >= wb2;
        const uint64_t ob = ballot(offer);
        if (offer) {
            FpsSlot& o = L.w.wl[wave][mbcnt(ob)];
            o.v = __int_as_float(b1);
            o.i = lbase + k1;
            o.c = make_float4(bx, by, bz, bt);
        }
        if (lane == 0) {
            L.w.wc[wave] = __popcll(ob);
            L.w.wb[wave] = wb2;
        }
        __syncthreads();
        int Uw = 0;
#pragma unroll
        for (int w = 0; w < kFpsW; ++w) Uw = max(Uw, (int)__builtin_amdgcn_readfirstlane(L.w.wb[w]));
        int rb = INT32_MIN, re = 0;
        int kcnt[kFpsW];
#pragma unroll
        for (int w = 0; w < kFpsW; ++w) {
            const int cw = __builtin_amdgcn_readfirstlane(L.w.wc[w]);
            const int v = lane < cw ? __float_as_int(L.w.wl[w][lane < cw ? lane : 0].v) : INT32_MIN;
            const bool g = v > rb;
            rb = g ? v : rb;
            re = g ? w : re;
            kcnt[w] = __popcll(ballot(v > Uw));
        }
        const int gm = wave_max_i(rb);
        int Lb, eb;
        {
            const uint64_t m = ballot(rb == gm);
            if (__popcll(m) == 1) {
                Lb = (int)__builtin_ctzll(m);
                eb = readlane_i(re, Lb);
            } else {
                const int f = wave_min_i(rb == gm ? re * 64 + lane : INT32_MAX);
                Lb = f & 63;
                eb = f >> 6;
            }
        }
        int base = 0, C = 0;
#pragma unroll
        for (int w = 0; w < kFpsW; ++w) {
            base += w < wave ? kcnt[w] : 0;
            C += kcnt[w];
        }
        const bool keep = offer && b1 > Uw;
        const int pos = base + mbcnt(ballot(keep));
        if (keep && pos < kRecSlots - 1) {
            FpsSlot& o = L.w.list[pos];
            o.v = __int_as_float(b1);
            o.i = lbase + k1;
            o.c = make_float4(bx, by, bz, bt);
        }
        if (C > kRecSlots - 1) {
            const int d = wave_max_i(keep && pos >= kRecSlots - 1 ? b1 : INT32_MIN);
            if (lane == 0) L.w.wd[wave] = d;
            __syncthreads();
#pragma unroll
            for (int w = 0; w < kFpsW; ++w) Uw = max(Uw, (int)__builtin_amdgcn_readfirstlane(L.w.wd[w]));
        }
        __syncthreads();

        // ---- 2. publish this shard's record
        const int tag = j + 1;
        const int par = ex & 1;
        // record of shard q: rec0 + q * 2 * kGangRecWords
        unsigned long long* rec0 = sh.rec + (size_t)par * kGangRecWords;
        if (wave == 0) {
            unsigned long long* r = rec0 + (size_t)sh.g * 2 * kGangRecWords;
            int ov = kNoEntry, oi = 0;
            if (lane == kRecSlots - 1) {
                const FpsSlot& o = L.w.wl[eb][Lb];
                ov = __float_as_int(o.v);
                oi = o.i;
            } else if (lane < C) {
                const FpsSlot& o = L.w.list[lane];
                ov = __float_as_int(o.v);
                oi = o.i;
            }
            rec_store(r + lane, rec_word(tag, oi, ov));
            if (lane == 0) rec_store(r + kRecBound, rec_word(tag, 0, Uw));
        }

        // ---- 3. read every shard's record
        // thread t reads record entries F = t + 256q (shard F/64, slot
        // F%64); threads t < G also the best pulse and the bound of shard t
        const int nF = G * kRecSlots;
        const int nq = (nF + kFpsT - 1) / kFpsT;  // read rounds in use (uniform)
        const char* rbase = reinterpret_cast<const char*>(rec0);
        unsigned long long vw[kGangQ];
        unsigned long long bw0 = 0, bw1 = 0;
        {
            const uint32_t so = (uint32_t)(tid < G ? tid : 0) * 2u * kGangRecWords * 8u;
            for (uint32_t spin = 0;; ++spin) {
                // every load of a spin is issued before any is tested, so a
                // spin costs one round trip: no load sits in a divergent
                // branch (lanes past the records re-read the last entry, and
                // threads t >= G the words of shard 0)
                // an opaque zero keeps the offsets from being hoisted out of
                // the wait loop (they are cheap; registers are not)
                int z;
                asm volatile("v_mov_b32 %0, 0" : "=v"(z));
#pragma unroll
                for (int q = 0; q < kGangQ; ++q) {
                    if (q < nq) {
                        const int F = min(tid + kFpsT * q + z, nF - 1);
                        const uint32_t o = ((uint32_t)(F >> 6) * 2u * kGangRecWords + (uint32_t)(F & 63)) * 8u;
                        vw[q] = rec_load(reinterpret_cast<const unsigned long long*>(rbase + o));
                    }
                }
                bw0 = rec_load(reinterpret_cast<const unsigned long long*>(rbase + so + (kRecSlots - 1) * 8u));
                bw1 = rec_load(reinterpret_cast<const unsigned long long*>(rbase + so + kRecBound * 8u));
                bool ok = rec_ok(bw0, tag) && rec_ok(bw1, tag);
#pragma unroll
                for (int q = 0; q < kGangQ; ++q)
                    if (q < nq) ok = ok && rec_ok(vw[q], tag);
                if (__syncthreads_and(ok)) break;
                if (spin >= sh.spin_limit) {
                    // give up: the exchange goes on with what it read, and the
                    // error word tells the caller the outputs are not valid
                    if (tid == 0)
                        __hip_atomic_fetch_or(sh.err, kErrFpsWait, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        // the gang's argmax and bound (wave 0 holds every shard's)
        if (wave == 0) {
            const bool has = lane < G;
            const int u = has ? rec_val(bw1) : 0;
            const int Ug = wave_max_i(u);
            const int v = has ? rec_val(bw0) : INT32_MIN;
            const int vm = wave_max_i(v);
            const int Lg = (int)__builtin_ctzll(ballot(has && v == vm));
            if (lane == Lg) {
                // the winner's coordinates are fetched now, overlapping the
                // list construction below
                const int wi = min(rec_idx(bw0), n - 1);
                L.gwin.v = __int_as_float(v);
                L.gwin.i = wi;
                L.gwin.c = p[wi];
            }
            if (lane == 0) L.gU = Ug;
        }
        __syncthreads();
        int Ug = __builtin_amdgcn_readfirstlane(L.gU);
#pragma unroll
        for (int q = 0; q < kGangQ; ++q) {
            const int F = tid + kFpsT * q;
            const bool kq = q < nq && F < nF && rec_val(vw[q]) > Ug;
            const uint64_t kb = ballot(kq);
            if (lane == 0) L.gcnt[q * kFpsW + wave] = __popcll(kb);
        }
        __syncthreads();
        // positions in (shard, slot) order = F order: round q, then wave,
        // then lane; an exclusive scan of the (q, wave) counts, one per lane
        static_assert(kGangQ * kFpsW == 64, "one count per lane");
        const int cnt_l = L.gcnt[lane];
        const int incl_l = wave_incl_scan(cnt_l);
        const int excl_l = incl_l - cnt_l;
        const int Cg = readlane_i(incl_l, 63);
        int dropped = INT32_MIN;
#pragma unroll
        for (int q = 0; q < kGangQ; ++q) {
            const int F = tid + kFpsT * q;
            const bool kq = q < nq && F < nF && rec_val(vw[q]) > Ug;
            const int gpos = readlane_i(excl_l, q * kFpsW + wave) + mbcnt(ballot(kq));
            if (kq && gpos < kGangCap) {
                FpsSlot& o = L.glist[gpos];
                o.v = __int_as_float(rec_val(vw[q]));
                o.i = min(rec_idx(vw[q]), n - 1);
            }
            dropped = kq && gpos >= kGangCap ? max(dropped, rec_val(vw[q])) : dropped;
        }
        if (Cg > kGangCap) {
            const int d = wave_max_i(dropped);
            if (lane == 0) L.gdrop[wave] = d;
            __syncthreads();
#pragma unroll
            for (int w = 0; w < kFpsW; ++w) Ug = max(Ug, (int)__builtin_amdgcn_readfirstlane(L.gdrop[w]));
        }
        __syncthreads();
        {
            const int gv = __builtin_amdgcn_readfirstlane(__float_as_int(L.gwin.v));
            if (gv <= 0) {
                s = min(first_unselected_lds(L.w.bm[wave], s_sel, selv, j), n - 1);
                const float4 q = p[s];
                cx = readlane_f(q.x, 0);
                cy = readlane_f(q.y, 0);
                cz = readlane_f(q.z, 0);
                ct = readlane_f(q.w, 0);
            } else {
                s = min(max((int)__builtin_amdgcn_readfirstlane(L.gwin.i), 0), n - 1);
                cx = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(L.gwin.c.x)));
                cy = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(L.gwin.c.y)));
                cz = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(L.gwin.c.z)));
                ct = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(L.gwin.c.w)));
            }
        }
        const int Cl = min(Cg, kGangCap);
        nreg = __builtin_amdgcn_readfirstlane((Cl + 63) >> 6);
        U = __builtin_amdgcn_readfirstlane(Ug);
        // the entries' coordinates come from the input, one gather per list
        // register, all in flight together: no gather sits behind a branch
        // (entries past the list read pulse 0 and stay unused)
#pragma unroll
        for (int e = 0; e < kGangE; ++e) {
            const int f = e * 64 + lane;
            const bool has = f < Cl;
            li[e] = has ? L.glist[f].i : 0;
            lv[e] = has ? L.glist[f].v : -1.0f;
        }
#pragma unroll
        for (int e = 0; e < kGangE; ++e) {
            const float4 q = p[li[e]];
            lx[e] = q.x;
            ly[e] = q.y;
            lz[e] = q.z;
            lt[e] = q.w;
        }
        ++ex;
        ++j;
    }
    if (wave == 0 && lane <= (j & 63)) s_sel[(j & ~63) + lane] = selv;
    if (a.assign) {
#pragma unroll
        for (int k = 0; k < M; ++k) {
            const int i = lbase + k;
            if (i < send) a.assign[off + i] = nr[k];
        }
    }
    if (s_asg) {
        __syncthreads();  // s_asg overlaps this function's LDS
#pragma unroll
        for (int k = 0; k < M; ++k) {
            const int i = lbase + k;
            if (i < send) s_asg[i - sh.lo] = nr[k];
        }
    }
    __builtin_amdgcn_s_setprio(0);
    if (sh.g == 0) write_selection(a, b, p, s_sel);
    return ex;
}

__device__ __forceinline__ int fps_gang_dispatch(const SampleArgs& a, int64_t b, int64_t off, int n,
                                                 int s0, const Shard& sh, GangLds& L, int* ss, int* sa) {
    switch ((sh.cnt + kFpsT - 1) / kFpsT) {
        case 1: case 2: case 3: case 4: case 5: case 6: case 7: case 8: case 9: case 10:
            return fps_gang<10>(a, b, off, n, s0, sh, L, ss, sa);
        case 11: case 12: return fps_gang<12>(a, b, off, n, s0, sh, L, ss, sa);
        case 13: case 14: return fps_gang<14>(a, b, off, n, s0, sh, L, ss, sa);
        default: return fps_gang<16>(a, b, off, n, s0, sh, L, ss, sa);
    }
}

// FPS of one event of any size by one workgroup, state streamed from the
// workspace (min distance) and from `assign` or the workspace (nearest slot)
// every iteration.  Used only for events beyond kGangMax * kFpsCap pulses.
// Thread t owns pulses t, t+256, ...; the argmax resolves ties by an
// explicit minimum over the index.
__device__ __forceinline__ void fps_streaming(const SampleArgs& a, int64_t b, int64_t off, int n, int s0,
                              FpsSlot (*slots)[kFpsW], int* s_sel) {
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int P = a.P;
    const float4* __restrict__ p = a.coords + off;
    float* __restrict__ mind = a.ws_mind + off;
    int32_t* __restrict__ nr = (a.assign ? a.assign : a.ws_near) + off;

    uint32_t selbits = 0;
    int s = s0;
    float4 c = p[s];
    for (int j = 0; j < P; ++j) {
        if (tid == 0) s_sel[j] = s;
        mark_selected(selbits, s);
        float bv = -1.0f;
        int bi = 0x7fffffff;
        for (int i = tid; i < n; i += kFpsT) {
            const float4 q = p[i];
            const float d = sqd(q.x, q.y, q.z, q.w, c.x, c.y, c.z, c.w);
            float mi = j == 0 ? INFINITY : mind[i];
            if (d < mi) {
                mi = d;
                mind[i] = d;
                nr[i] = j;
            } else if (j == 0) {
                mind[i] = mi;
                nr[i] = 0;
            }
            if (mi > bv) {
                bv = mi;
                bi = i;
            }
        }
        if (j + 1 == P) break;
        const float wm = __int_as_float(wave_max_i(__float_as_int(bv)));
        const int wi = wave_min_i(bv == wm ? bi : 0x7fffffff);
        if (lane == 0) {
            FpsSlot& o = slots[j & 1][wave];
            o.v = wm;
            o.i = wi;
        }
        __syncthreads();
        // largest value, then smallest index
        const bool has = lane < kFpsW;
        FpsSlot sl;
        if (has) sl = slots[j & 1][lane];
        const int v = has ? __float_as_int(sl.v) : INT32_MIN;
        int r = max(v, dpp_i<kQuadSwap1, 0xF>(v, INT32_MIN));
        r = max(r, dpp_i<kQuadSwap2, 0xF>(r, INT32_MIN));
        const float gm = __int_as_float(readlane_i(r, 0));
        const int gi = wave_min_i(has && v == __float_as_int(gm) ? sl.i : 0x7fffffff);
        s = gm == 0.0f ? first_unselected(selbits) : gi;
        s = min(max(s, 0), n - 1);
        c = p[s];
    }
    write_selection(a, b, p, s_sel);
}

// Work list of the sample call, built by one workgroup (up to 1024 threads):
// first every shard of every event that needs a gang (kFpsCap < n <=
// kGangMax*kFpsCap; shards of one event consecutive), then one item per other
// event.  Zeroes the gang records and the claim counter.  header[5] receives
// the number of gang items: when it is 0, item i is event i and the sample
// workgroups take their items by workgroup index instead of claiming them.
__device__ __forceinline__ void plan_fps(const SampleArgs& a, int64_t B) {
    __shared__ int s_wsum[2][16];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int nt = (int)blockDim.x;  // a multiple of 64, at most 1024
    const int nw = nt >> 6;
    const int64_t max_items = B + a.N / kFpsCap;
    // malformed (overlapping) offsets could ask for more items than the list
    // holds; those are dropped, never written out of bounds
    auto put = [&](int64_t pos, int cnt, int64_t b) {
        for (int q = 0; q < cnt && pos + q < max_items; ++q) {
            a.item_ev[pos + q] = (int32_t)b;
            a.item_g[pos + q] = q;
        }
    };
    int gang_items = 0, items = 0;
    if (B <= nt) {
        // one pass: both counts of event `tid` and their two scans
        int gc = 0, sc = 0;
        if (tid < B) {
            int64_t off;
            int n;
            event_range(a.offsets, a.N, tid, off, n);
            const bool gang = n > kFpsCap && n <= kGangMax * kFpsCap && n > a.P;
            gc = gang ? (n + kFpsCap - 1) / kFpsCap : 0;
            sc = gang ? 0 : 1;
        }
        const int gi = wave_incl_scan(gc);
        const int si = wave_incl_scan(sc);
        if (lane == 63) {
            s_wsum[0][wave] = gi;
            s_wsum[1][wave] = si;
        }
        __syncthreads();
        int gb = 0, sb = 0;
        for (int w = 0; w < nw; ++w) {
            const int g = s_wsum[0][w], v = s_wsum[1][w];
            if (w < wave) {
                gb += g;
                sb += v;
            }
            gang_items += g;
            items += v;
        }
        items += gang_items;
        put(gb + gi - gc, gc, tid);
        put(gang_items + sb + si - sc, sc, tid);
    } else {
        int carry = 0;
        for (int pass = 0; pass < 2; ++pass) {
            for (int64_t base = 0; base < B; base += nt) {
                const int64_t b = base + tid;
                int cnt = 0;
                if (b < B) {
                    int64_t off;
                    int n;
                    event_range(a.offsets, a.N, b, off, n);
                    const bool gang = n > kFpsCap && n <= kGangMax * kFpsCap && n > a.P;
                    if (pass == 0 && gang) cnt = (n + kFpsCap - 1) / kFpsCap;
                    if (pass == 1 && !gang) cnt = 1;
                }
                const int incl = wave_incl_scan(cnt);
                if (lane == 63) s_wsum[0][wave] = incl;
                __syncthreads();
                int wb = 0, total = 0;
                for (int w = 0; w < nw; ++w) {
                    const int v = s_wsum[0][w];
                    if (w < wave) wb += v;
                    total += v;
                }
                put(carry + wb + incl - cnt, cnt, b);
                carry += total;
                __syncthreads();
            }
            if (pass == 0) gang_items = carry;
        }
        items = carry;
    }
    // gang items come first: clear their records (stale tags of an earlier
    // call must not match)
    gang_items = (int)min((int64_t)gang_items, max_items);
    // 16-byte stores (a gang item's records are 2 * kGangRecWords 64-bit
    // words, an even count, from a 256-byte aligned base)
    static_assert(kGangRecWords % 2 == 0, "records clear in 16-byte stores");
    const int64_t gw = (int64_t)gang_items * kGangRecWords;
    uint4* rec4 = reinterpret_cast<uint4*>(a.gang_rec);
    for (int64_t w = tid; w < gw; w += nt) rec4[w] = make_uint4(0u, 0u, 0u, 0u);
    if (tid == 0) {
        a.header[1] = (int)min((int64_t)items, max_items);  // items
        a.header[2] = 0;                                   // claim counter
        a.header[3] = 0;                                   // device error word
        a.header[5] = gang_items;
    }
}

__global__ __launch_bounds__(1024) void plan_fps_kernel(SampleArgs a, int64_t B) {
    plan_fps(a, B);
}

// The work lists of a call that runs sample, then Lloyd (assign chunks,
// when `chunks`) and Voronoi pooling (pooling chunks, when `pool`), in one
// launch.
template <bool kBands>
__global__ __launch_bounds__(1024) void plan_all_kernel(SampleArgs a, int64_t B,
                                                        int32_t* __restrict__ chunk_ev,
                                                        int32_t* __restrict__ chunk_beg,
                                                        int64_t max_chunks, PoolArgs pa,
                                                        int64_t max_pool_chunks,
                                                        int64_t max_parts, int chunks, int pool,
                                                        int64_t band_over) {
    if (!a.direct) plan_fps(a, B);  // no work list in direct mode
    if (chunks) {
        __syncthreads();
        plan_chunks(a.offsets, B, a.N, max_chunks, a.header, chunk_ev, chunk_beg);
    }
    if (pool) {
        __syncthreads();
        plan_pool<kBands>(a.offsets, B, a.N, max_pool_chunks, max_parts, pa.header,
                  const_cast<int32_t*>(pa.chunk_ev), const_cast<int32_t*>(pa.chunk_beg),
                  const_cast<int32_t*>(pa.chunk_part), const_cast<int32_t*>(pa.big_ev),
                  pa.whole, band_over);
    }
}

// What one workgroup did for its work item, for the fused pooling that may
// follow.
struct ItemInfo {
    int64_t b;    // event (-1: no item)
    int64_t off;  // first row of the event
    int n;        // pulses of the event
    int kind;     // 0 pass-through, 1 single workgroup, 2 gang shard, 3 streaming
    int g, G;     // shard and shards (gangs)
    int lo, cnt;  // the shard's pulses
    int item0;    // work item of shard 0 (gangs)
    int par;      // gang record parity no shard reads any more (gangs)
    bool staged;  // the event's feature rows were staged in LDS (single workgroup)
    bool deferred;  // the selection is left to the caller (staged, bitmap-sortable)
};

// Claim one work item and run FPS (or pass-through) for it.  s_asg, when not
// null, receives the shard's Voronoi slots (register-resident paths only).
// With `feats` given, a single-workgroup event of at most stage_cap feature
// floats also gets its C-column feature rows copied to s_feat.
template <bool kDirect>
__device__ __forceinline__ ItemInfo sample_item(const SampleArgs& a, int* s_item,
                                                FpsSlot (*s_slots)[kFpsW], GangLds& s_gang,
                                                int* s_sel, int* s_asg, const float* feats, int C,
                                                int stage_cap, float* s_feat) {
    const int tid = threadIdx.x;
    ItemInfo it{-1, 0, 0, 0, 0, 1, 0, 0, 0, 0, false, false};
    // without gangs item i is event i: the event's range is read together
    // with the header, and nothing is claimed; in direct mode (no work list
    // was planned) the header is not read at all
    const int64_t bd = (int64_t)blockIdx.x < a.B ? (int64_t)blockIdx.x : a.B - 1;
    int64_t off;
    int n;
    event_range(a.offsets, a.N, bd, off, n);
    int item;
    int64_t b;
    int g;
    if (kDirect || a.direct) {
        item = (int)blockIdx.x;
        if (item >= a.B) return it;
        b = item;
        g = 0;
    } else if (a.header[5] == 0) {
        const int nitems = a.header[1];
        item = (int)blockIdx.x;
        if (item >= nitems) return it;
        b = item;
        g = 0;
    } else {
        const int nitems = a.header[1];
        // items are claimed in list order, so the shards of one gang go to
        // workgroups that start one after another: a gang whose workgroups
        // wait for a partner only ever waits for a workgroup that will start
        // once earlier, complete gangs or single events finish
        if (tid == 0)
            *s_item = __hip_atomic_fetch_add(a.header + 2, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        item = *s_item;
        if (item >= nitems) return it;
        b = a.item_ev[item];
        g = a.item_g[item];
        event_range(a.offsets, a.N, b, off, n);
    }
    it.b = b;
    it.off = off;
    it.n = n;
    it.g = g;
    it.item0 = item - g;
    const int P = a.P;
    if (n <= P) {
        // small events keep one token per pulse
        for (int j = tid; j < P; j += kFpsT) {
            if (j < n) {
                a.centroid_idx[b * P + j] = j;
                a.centroids[b * P + j] = a.coords[off + j];
                if (a.assign) a.assign[off + j] = j;
            } else {
                a.centroid_idx[b * P + j] = -1;
                a.centroids[b * P + j] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        if (tid == 0) a.token_count[b] = n;
        it.kind = 0;
        it.cnt = n;
        return it;
    }
    int s0 = a.start_idx ? a.start_idx[b] : 0;
    if (s0 < 0 || s0 >= n) s0 = 0;
    if (n <= kFpsCap) {
        it.staged = feats != nullptr && (int64_t)(n + 1) * C <= stage_cap;
        // a staged event that the fused tail sorts through bitmaps writes its
        // selection there, after the pooling (the coordinates' loads then
        // overlap the sort)
        it.deferred = it.staged && n <= kBmW4 * 128 && P * ((n + 127) >> 7) <= kFpsCap / 4;
        const Stage st{it.staged ? feats + off * C : nullptr, it.staged ? n * C : 0,
                       it.staged ? (n + 1) * C : 0, s_feat, it.deferred ? 1 : 0};
        fps_single_dispatch(a, b, off, n, s0, *reinterpret_cast<SingleLds*>(&s_gang), s_sel,
                            s_asg, st);
        it.kind = 1;
        it.cnt = n;
    } else if (!kDirect && !a.direct && n <= kGangMax * kFpsCap) {
        const int G = (n + kFpsCap - 1) / kFpsCap;
        const int S = (n + G - 1) / G;
        const int lo = g * S;
        const Shard sh{lo, min(S, n - lo), g, G,
                       a.gang_rec + (size_t)(item - g) * 2 * kGangRecWords, a.header + 3,
                       a.spin_limit};
        it.par = fps_gang_dispatch(a, b, off, n, s0, sh, s_gang, s_sel, s_asg) & 1;
        it.kind = 2;
        it.G = G;
        it.lo = lo;
        it.cnt = sh.cnt;
    } else {
        fps_streaming(a, b, off, n, s0, s_slots, s_sel);
        it.kind = 3;
        it.cnt = n;
    }
    if (tid == 0 && g == 0) a.token_count[b] = P;
    return it;
}

__global__ __launch_bounds__(kFpsT) void sample_kernel(SampleArgs a) {
    // in direct mode no planner clears the device error word (nothing in
    // this mode can set it)
    if (a.direct && blockIdx.x == 0 && threadIdx.x == 0) a.header[3] = 0;
    __shared__ int s_item;
    __shared__ FpsSlot s_slots[2][kFpsW];
    __shared__ int s_sel[FPSTOK_MAX_SLOTS];
    __shared__ GangLds s_gang;
    sample_item<false>(a, &s_item, s_slots, s_gang, s_sel, nullptr, nullptr, 0, 0, nullptr);
}

// ------------------------------------------------------------------- assign

constexpr int kAsgT = 256;
constexpr int kAsgQ = 4;  // threads per pulse, each over a quarter of the centroids
static_assert(kChunk * kAsgQ == kAsgT, "one chunk per workgroup");

// Nearest centroid of every pulse of one chunk (kChunk pulses), lowest slot
// on ties.  Centroids are staged in LDS.  The kAsgQ threads of a pulse (a
// quad of lanes) each scan a contiguous quarter of the centroids in
// ascending order with a strict comparison, then merge across the quad
// (two DPP steps): the lower quarter wins ties, so the result is the first
// minimum over all centroids.
__global__ __launch_bounds__(kAsgT) void assign_kernel(AssignArgs a) {
    __shared__ float4 s_c[1024];
    // the chunk's description is read together with the chunk count (the
    // grid has max_chunks workgroups, so the read is in bounds), and the
    // event's P centroid rows together with its range and token count:
    // three dependent rounds of loads instead of five
    const int w = blockIdx.x;
    const int nchunks = a.header[0];
    const int64_t b = a.chunk_ev[w];
    const int beg = a.chunk_beg[w];
    if (w >= nchunks) return;
    int64_t off;
    int n;
    event_range(a.offsets, a.N, b, off, n);
    int T = a.token_count[b];
    const int tid = threadIdx.x;
    float4 cv[1024 / kAsgT];
#pragma unroll
    for (int r = 0; r < 1024 / kAsgT; ++r) {
        cv[r] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r * kAsgT < a.P) cv[r] = a.centroids[b * a.P + min(tid + r * kAsgT, a.P - 1)];
    }
    if (n == 0 || (a.skip_small && n <= a.P)) return;
    T = T > a.P ? a.P : T;
    if (T < 1) return;
#pragma unroll
    for (int r = 0; r < 1024 / kAsgT; ++r)
        if (r * kAsgT < a.P && tid + r * kAsgT < T) s_c[tid + r * kAsgT] = cv[r];
    __syncthreads();
    const int q = tid & (kAsgQ - 1);
    const int i = beg + (tid >> 2);
    const int end = min(n, beg + kChunk);
    float4 p = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < end) p = a.coords[off + i];
    const int T4 = (T + kAsgQ - 1) >> 2;
    const int j0 = min(T, q * T4), j1 = min(T, j0 + T4);
    float bd = INFINITY;
    int bj = j0;
    for (int j = j0; j < j1; ++j) {
        const float4 c = s_c[j];
        const float d = sqd(p.x, p.y, p.z, p.w, c.x, c.y, c.z, c.w);
        const bool u = d < bd;
        bd = u ? d : bd;
        bj = u ? j : bj;
    }
    // merge the quad: partner q^1, then q^2; the lower quarter comes first
#pragma unroll
    for (int step = 0; step < 2; ++step) {
        const int od = step == 0 ? dpp_i<kQuadSwap1, 0xF>(__float_as_int(bd), 0)
                                 : dpp_i<kQuadSwap2, 0xF>(__float_as_int(bd), 0);
        const int oj = step == 0 ? dpp_i<kQuadSwap1, 0xF>(bj, 0) : dpp_i<kQuadSwap2, 0xF>(bj, 0);
        const bool lower = ((q >> step) & 1) == 0;  // this lane holds the lower range
        const float ad = lower ? bd : __int_as_float(od);
        const int aj = lower ? bj : oj;
        const float xd = lower ? __int_as_float(od) : bd;
        const int xj = lower ? oj : bj;
        const bool tb = xd < ad;
        bd = tb ? xd : ad;
        bj = tb ? xj : aj;
    }
    if (q == 0 && i < end) a.assign[off + i] = bj;
}

// ---------------------------------------------------------------------- kNN

constexpr int kKnnT = 256;
constexpr int kKnnW = kKnnT / 64;
constexpr int kKnnCap = 512;  // candidates per wave held in LDS
constexpr int kKnnPoolB = 8;  // list members whose rows are loaded together when pooling
constexpr int kKnnReg = 8;    // keys per lane kept in registers (events of up to 512 pulses)

__device__ __forceinline__ uint64_t dkey(float d, int i) {
    return ((uint64_t)__float_as_uint(d) << 32) | (uint32_t)i;
}

// One wave per (event, token): the k smallest (d2, index) keys.
//  1. Each lane finds its own smallest key; the k-th smallest of these 64
//     lane minima is an upper bound tau on the k-th smallest key overall
//     (they are k distinct pulses).
//  2. Every key <= tau is collected into LDS (usually about k of them).
//  3. The candidates are ranked by counting and the first k written out.
//  If more than kKnnCap keys are <= tau, k rounds of wave-wide
//  min-extraction are used instead.
// The members of token j's list, pooled in list order by the wave that
// ranked them: lane c sums column c (and every lane the weights) in float64,
// as the kNN pooling kernel does; members are loaded kBatch at a time with
// clamped indices (no load behind a per-lane branch).
__device__ __forceinline__ void knn_pool_list(const KnnArgs& a, int64_t b, int64_t off, int n,
                                              int j, int len, const int* lst) {
    const int lane = lane_id();
    const int C = a.C;
    float* __restrict__ out = a.pooled + (b * a.P + j) * (int64_t)C;
    for (int c0 = 0; c0 < C; c0 += 64) {
        const int c = c0 + lane;
        const int cc = c < C ? c : C - 1;
        double W = 0.0, S = 0.0;
        for (int m0 = 0; m0 < len; m0 += kKnnPoolB) {
            int idx[kKnnPoolB];
            float w[kKnnPoolB], f[kKnnPoolB];
#pragma unroll
            for (int q = 0; q < kKnnPoolB; ++q) {
                const int i = lst[min(m0 + q, len - 1)];
                idx[q] = m0 + q < len && i >= 0 && i < n ? i : -1;
            }
#pragma unroll
            for (int q = 0; q < kKnnPoolB; ++q) {
                const float* __restrict__ r = a.features + (off + (idx[q] >= 0 ? idx[q] : 0)) * (int64_t)C;
                w[q] = a.weight_col >= 0 ? r[a.weight_col] : 1.0f;
                f[q] = r[cc];
            }
#pragma unroll
            for (int q = 0; q < kKnnPoolB; ++q) {
                if (idx[q] >= 0) {
                    const double wd = (double)w[q];
                    W += wd;
                    S += wd * (double)f[q];
                }
            }
        }
        if (c < C) out[c] = W != 0.0 ? (float)(S / W) : 0.0f;
    }
    if (a.cell_count && lane == 0) {
        int count = 0;
        for (int e = 0; e < len; ++e) count += (lst[e] >= 0 && lst[e] < n) ? 1 : 0;
        a.cell_count[b * a.P + j] = count;
    }
}

__global__ __launch_bounds__(kKnnT) void knn_kernel(KnnArgs a) {
    __shared__ uint64_t s_buf[kKnnW][kKnnCap];
    __shared__ int s_lst[kKnnW][kKnnMaxK];
    const int P = a.P;
    const int k = a.k;
    const int nb = (P + kKnnW - 1) / kKnnW;
    const int64_t b = blockIdx.x / nb;
    const int wave = threadIdx.x >> 6;
    const int lane = lane_id();
    const int j = (int)(blockIdx.x % nb) * kKnnW + wave;
    if (j >= P) return;
    int64_t off;
    int n;
    event_range(a.offsets, a.N, b, off, n);
    int T = a.token_count[b];
    T = T < 0 ? 0 : (T > P ? P : T);
    int32_t* __restrict__ row = a.knn_idx + (b * P + j) * (int64_t)k;
    int* lst = s_lst[wave];
    if (j >= T || n <= P) {
        for (int e = lane; e < k; e += 64) {
            const int v = (e == 0 && j < T && j < n) ? j : -1;
            row[e] = v;
            lst[e] = v;
        }
        if (a.pooled) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // only the list's first entry can be a pulse
            knn_pool_list(a, b, off, n, j, j < T && j < n ? 1 : 0, lst);
        }
        return;
    }
    const float4 c = a.centroids[b * P + j];
    const float4* __restrict__ p = a.coords + off;

    // events of up to kKnnReg * 64 pulses keep their keys in registers
    // (lane l: pulses l, l+64, ...), loaded together with clamped indices,
    // so both passes below read the coordinates once
    const bool inreg = n <= kKnnReg * 64;
    uint64_t keys[kKnnReg];
    uint64_t mykey = ~0ull;
    if (inreg) {
        float4 qs[kKnnReg];
#pragma unroll
        for (int r = 0; r < kKnnReg; ++r) qs[r] = p[min(r * 64 + lane, n - 1)];
#pragma unroll
        for (int r = 0; r < kKnnReg; ++r) {
            const int i = r * 64 + lane;
            keys[r] = i < n ? dkey(sqd(qs[r].x, qs[r].y, qs[r].z, qs[r].w, c.x, c.y, c.z, c.w), i)
                            : ~0ull;
            mykey = keys[r] < mykey ? keys[r] : mykey;
        }
    } else {
        for (int i = lane; i < n; i += 64) {
            const float4 q = p[i];
            const uint64_t key = dkey(sqd(q.x, q.y, q.z, q.w, c.x, c.y, c.z, c.w), i);
            mykey = key < mykey ? key : mykey;
        }
    }
    const int valid = min(n, 64);
    uint64_t tau = ~0ull;
    if (k <= valid) {
        // the k-th smallest distance word (a key's high half) among the lane
        // minima, bit by bit from the top: the smallest t with at least k
        // lane minima at or below it.  Every key whose distance is at most t
        // qualifies, so tau bounds the k-th smallest key from above (keys of
        // equal distance only add candidates, which the exact ranking below
        // orders).
        const uint32_t hi = (uint32_t)(mykey >> 32);
        uint32_t t = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t below = t | ((1u << bit) - 1u);  // this bit 0, the lower ones 1
            if (__popcll(ballot(hi <= below)) < k) t |= 1u << bit;
        }
        tau = ((uint64_t)t << 32) | 0xFFFFFFFFull;
    }
    uint64_t* __restrict__ buf = s_buf[wave];
    int cnt = 0;
    if (inreg) {
#pragma unroll
        for (int r = 0; r < kKnnReg; ++r) {
            if (r * 64 < n) {
                const int i = r * 64 + lane;
                const uint64_t key = keys[r];
                const bool take = i < n && key <= tau;
                const uint64_t bl = ballot(take);
                const int pos = cnt + mbcnt(bl);
                if (take && pos < kKnnCap) buf[pos] = key;
                cnt += __popcll(bl);
            }
        }
    } else {
        for (int i0 = 0; i0 < n; i0 += 64) {
            const int i = i0 + lane;
            uint64_t key = ~0ull;
            if (i < n) {
                const float4 q = p[i];
                key = dkey(sqd(q.x, q.y, q.z, q.w, c.x, c.y, c.z, c.w), i);
            }
            const bool take = i < n && key <= tau;
            const uint64_t bl = ballot(take);
            const int pos = cnt + mbcnt(bl);
            if (take && pos < kKnnCap) buf[pos] = key;
            cnt += __popcll(bl);
        }
    }
    const int need = min(k, n);
    if (cnt <= kKnnCap) {
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        for (int q = lane; q < cnt; q += 64) {
            const uint64_t kq = buf[q];
            int rank = 0;
            for (int r = 0; r < cnt; ++r) rank += buf[r] < kq ? 1 : 0;
            if (rank < k) {
                row[rank] = (int)(uint32_t)kq;
                lst[rank] = (int)(uint32_t)kq;
            }
        }
    } else {
        // k rounds of extracting the smallest key above the previous one
        uint64_t last = 0;
        for (int e = 0; e < need; ++e) {
            uint64_t best = ~0ull;
            for (int i = lane; i < n; i += 64) {
                const float4 q = p[i];
                const uint64_t key = dkey(sqd(q.x, q.y, q.z, q.w, c.x, c.y, c.z, c.w), i);
                if ((e == 0 || key > last) && key < best) best = key;
            }
            // wave minimum of a 64-bit key: high word first, then low word
            const uint32_t hi = (uint32_t)(best >> 32);
            const int mhi = wave_min_i((int)(hi ^ 0x80000000u)) ^ (int)0x80000000u;
            const uint32_t lo = (uint32_t)best;
            const bool cand = hi == (uint32_t)mhi;
            const int mlo = wave_min_i(cand ? (int)(lo ^ 0x80000000u) : 0x7fffffff) ^ (int)0x80000000u;
            last = ((uint64_t)(uint32_t)mhi << 32) | (uint32_t)mlo;
            if (lane == 0) {
                row[e] = (int)(uint32_t)last;
                lst[e] = (int)(uint32_t)last;
            }
        }
    }
    for (int e = need + lane; e < k; e += 64) {
        row[e] = -1;
        lst[e] = -1;
    }
    if (a.pooled) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        knn_pool_list(a, b, off, n, j, k, lst);
    }
}

// ---------------------------------------------------- stable sort by token

constexpr int kSortT = 256;
constexpr int kSortW = kSortT / 64;
constexpr int kMaxP = 1024;
constexpr int kMaxBits = 10;  // bits of a slot index below kMaxP
constexpr int kLdsPerm = 4096;  // events up to this size keep their permutation in LDS
constexpr int kBatch = 8;       // members whose loads are issued together

// Workgroup-wide stable counting sort of one event's pulses by slot:
// perm[s_off[j] + r] = the r-th pulse (ascending) with asg = j.  Pulses whose
// slot is outside [0, T) are left out.  Wave w handles the contiguous segment
// [w*seg, (w+1)*seg); inside a 64-pulse tile the rank of a pulse among equal
// slots comes from a bitwise ballot match, so the order is stable without
// atomics.  Two passes: count per (wave, slot), then place.  `perm` may point
// to LDS or to device memory.
//   s_cnt: LDS int[kSortW * kMaxP];  s_off: LDS int[kMaxP + 1]
// kAtomicCount: the counting pass adds with LDS atomics (the order of the
// counts does not matter) and the placing pass unrolls its key bits; used
// where it measured faster (the pooling backward), the plain form elsewhere.
template <bool kAtomicCount = false>
__device__ __forceinline__ void block_sort_by_token(const int32_t* __restrict__ asg, int n, int T,
                                                    int* __restrict__ perm, int* s_cnt,
                                                    int* s_off) {
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    int nbits = 0;
    while ((1 << nbits) < T) ++nbits;
    for (int q = tid; q < kSortW * T; q += kSortT) s_cnt[q] = 0;
    __syncthreads();
    const int seg = ((n + kSortW - 1) / kSortW + 63) & ~63;
    const int sbeg = wave * seg;
    const int send = min(n, sbeg + seg);
    int* __restrict__ wc = s_cnt + wave * T;

    for (int pass = 0; pass < 2; ++pass) {
        if (kAtomicCount && pass == 0) {
            for (int i = sbeg + lane; i < send; i += 64) {
                const int key = asg[i];
                if (key >= 0 && key < T) atomicAdd(&wc[key], 1);
            }
        } else if (kAtomicCount) {
            for (int t0 = sbeg; t0 < send; t0 += 64) {
                const int i = t0 + lane;
                const int key = i < send ? asg[i] : -1;
                const bool valid = key >= 0 && key < T;
                const uint64_t act = ballot(valid);
                uint32_t mlo = (uint32_t)act, mhi = (uint32_t)(act >> 32);
#pragma unroll
                for (int bit = 0; bit < kMaxBits; ++bit) {
                    if (bit < nbits) {
                        const bool bb = ((key >> bit) & 1) != 0;
                        const uint64_t bal = ballot(valid && bb);
                        const uint64_t nb = act & ~bal;
                        mlo &= bb ? (uint32_t)bal : (uint32_t)nb;
                        mhi &= bb ? (uint32_t)(bal >> 32) : (uint32_t)(nb >> 32);
                    }
                }
                const uint64_t match = ((uint64_t)mhi << 32) | mlo;
                const int rank = mbcnt(match);
                const int cnt = __popcll(match);
                if (valid) perm[wc[key] + rank] = i;
                __builtin_amdgcn_wave_barrier();
                if (valid && rank == 0) wc[key] += cnt;
                __builtin_amdgcn_wave_barrier();
            }
        } else {
            for (int t0 = sbeg; t0 < send; t0 += 64) {
                const int i = t0 + lane;
                int key = i < send ? asg[i] : -1;
                const bool valid = key >= 0 && key < T;
                const uint64_t act = ballot(valid);
                uint64_t match = act;
                for (int bit = 0; bit < nbits; ++bit) {
                    const bool bb = (key >> bit) & 1;
                    const uint64_t bal = ballot(valid && bb);
                    match &= bb ? bal : (act & ~bal);
                }
                const int rank = mbcnt(match);
                const int cnt = __popcll(match);
                if (pass == 1 && valid) perm[wc[key] + rank] = i;
                __builtin_amdgcn_wave_barrier();
                if (valid && rank == 0) wc[key] += cnt;
                __builtin_amdgcn_wave_barrier();
            }
        }
        __syncthreads();
        if (pass == 0) {
            // per slot: total over waves, exclusive scan over slots, then the
            // starting position of every (wave, slot) run
            int tot[kMaxP / kSortT];
            int local = 0;
            const int per = (T + kSortT - 1) / kSortT;
            for (int r = 0; r < per; ++r) {
                const int jj = tid * per + r;
                int t = 0;
                if (jj < T)
                    for (int w = 0; w < kSortW; ++w) t += s_cnt[w * T + jj];
                tot[r] = t;
                local += t;
            }
            __shared__ int s_wsum[kSortW];
            const int incl = wave_incl_scan(local);
            if (lane == 63) s_wsum[wave] = incl;
            __syncthreads();
            int run = incl - local;
            for (int w = 0; w < wave; ++w) run += s_wsum[w];
            int total = 0;
            for (int w = 0; w < kSortW; ++w) total += s_wsum[w];
            __syncthreads();
            for (int r = 0; r < per; ++r) {
                const int jj = tid * per + r;
                if (jj < T) {
                    s_off[jj] = run;
                    int pos = run;
                    for (int w = 0; w < kSortW; ++w) {
                        const int v = s_cnt[w * T + jj];
                        s_cnt[w * T + jj] = pos;
                        pos += v;
                    }
                }
                run += tot[r];
            }
            if (tid == 0) s_off[T] = total;
            __syncthreads();
        }
    }
}

constexpr int kSmallSlot = 64;  // largest slot block_sort_small handles
constexpr int kRankPer = kLdsPerm / kSortT;  // members one thread ranks at most

// The same stable sort, for the usual case of small slots and an LDS input
// that may be overwritten: counts and positions with LDS atomics (any order
// inside a slot, into `tmp`), then every member's rank inside its slot (the
// members of the slot with a lower pulse index) counted in parallel, and the
// members written to their final places -- into `asg` itself.  Returns
// false, with asg untouched, if some slot holds more than kSmallSlot pulses.
//   asg: LDS int[n] (n <= kLdsPerm);  tmp: LDS int[n];  s_cnt: LDS int[T];
//   s_off: LDS int[T + 1]
__device__ __forceinline__ bool block_sort_small(int* asg, int n, int T, int* tmp, int* s_cnt,
                                                 int* s_off) {
    __shared__ int s_ws[kSortW], s_wm[kSortW];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    for (int q = tid; q < T; q += kSortT) s_cnt[q] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kSortT) {
        const int k = asg[i];
        if (k >= 0 && k < T) atomicAdd(&s_cnt[k], 1);
    }
    __syncthreads();
    // exclusive scan of the counts (thread t: slots t*per .. t*per+per-1),
    // and the largest count
    const int per = (T + kSortT - 1) / kSortT;
    int loc[kMaxP / kSortT];
    int local = 0, mx = 0;
#pragma unroll
    for (int r = 0; r < kMaxP / kSortT; ++r) {
        const int jj = tid * per + r;
        const int c = r < per && jj < T ? s_cnt[jj] : 0;
        loc[r] = c;
        local += c;
        mx = max(mx, c);
    }
    const int incl = wave_incl_scan(local);
    const int wmx = wave_max_i(mx);
    if (lane == 63) s_ws[wave] = incl;
    if (lane == 0) s_wm[wave] = wmx;
    __syncthreads();
    int run = incl - local, total = 0, gmax = 0;
#pragma unroll
    for (int w = 0; w < kSortW; ++w) {
        const int v = s_ws[w];
        run += w < wave ? v : 0;
        total += v;
        gmax = max(gmax, s_wm[w]);
    }
    __syncthreads();
    if (gmax > kSmallSlot || n > kLdsPerm) return false;
#pragma unroll
    for (int r = 0; r < kMaxP / kSortT; ++r) {
        const int jj = tid * per + r;
        if (r < per && jj < T) {
            s_off[jj] = run;
            s_cnt[jj] = run;
        }
        run += loc[r];
    }
    if (tid == 0) s_off[T] = total;
    __syncthreads();
    for (int i = tid; i < n; i += kSortT) {
        const int k = asg[i];
        if (k >= 0 && k < T) tmp[atomicAdd(&s_cnt[k], 1)] = i;
    }
    __syncthreads();
    int dst[kRankPer], val[kRankPer];
#pragma unroll
    for (int r = 0; r < kRankPer; ++r) {
        const int x = tid + r * kSortT;
        dst[r] = -1;
        val[r] = 0;
        if (x < total) {
            const int v = tmp[x];
            const int j = asg[v];
            const int b0 = s_off[j], e0 = s_off[j + 1];
            int rank = 0;
            for (int y = b0; y < e0; ++y) rank += tmp[y] < v ? 1 : 0;
            dst[r] = b0 + rank;
            val[r] = v;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRankPer; ++r)
        if (dst[r] >= 0) asg[dst[r]] = val[r];
    __syncthreads();
    return true;
}

// Stable sort of a small event's pulses by slot through per-slot bitmaps
// (bit i of row k: pulse i has slot k).  A pulse's rank among its slot's
// members is the number of set bits of the row below its own, read from a
// prefix of popcounts per 128-bit word plus one masked word, so the order
// is ascending by construction, with no atomics on the order and no
// per-member loops.  perm[s_off[k] + r] = r-th member of slot k.
//   bm: LDS uint32[T * W4 * 4], W4 = ceil(n / 128) <= kW4Max;  pre4: LDS
//   int[T * W4];  s_off: LDS int[T + 1];  perm: LDS int[n]
template <int kW4Max = kBmW4>
__device__ __forceinline__ void block_sort_bitmap(const int* __restrict__ asg, int n, int T,
                                                  uint32_t* bm, int* pre4, int* s_off,
                                                  int* perm) {
    __shared__ int s_ws[kSortW];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int W4 = (n + 127) >> 7;
    uint4* bm4 = reinterpret_cast<uint4*>(bm);
    for (int q = tid; q < T * W4; q += kSortT) bm4[q] = make_uint4(0u, 0u, 0u, 0u);
    lds_barrier();
    for (int i = tid; i < n; i += kSortT) {
        const int k = asg[i];
        if ((unsigned)k < (unsigned)T) atomicOr(&bm[k * W4 * 4 + (i >> 5)], 1u << (i & 31));
    }
    lds_barrier();
    // slot jj (threads own `per` consecutive slots): prefix popcounts of its
    // row and its member count; then the exclusive scan of the counts
    const int per = (T + kSortT - 1) / kSortT;
    int loc[kMaxP / kSortT];
    int local = 0;
#pragma unroll
    for (int r = 0; r < kMaxP / kSortT; ++r) {
        const int jj = tid * per + r;
        int c = 0;
        if (r < per && jj < T) {
#pragma unroll
            for (int w4 = 0; w4 < kW4Max; ++w4) {
                if (w4 < W4) {
                    const uint4 q = bm4[jj * W4 + w4];
                    pre4[jj * W4 + w4] = c;
                    c += __popc(q.x) + __popc(q.y) + __popc(q.z) + __popc(q.w);
                }
            }
        }
        loc[r] = c;
        local += c;
    }
    const int incl = wave_incl_scan(local);
    if (lane == 63) s_ws[wave] = incl;
    lds_barrier();
    int run = incl - local, total = 0;
#pragma unroll
    for (int w = 0; w < kSortW; ++w) {
        const int v = s_ws[w];
        run += w < wave ? v : 0;
        total += v;
    }
#pragma unroll
    for (int r = 0; r < kMaxP / kSortT; ++r) {
        const int jj = tid * per + r;
        if (r < per && jj < T) s_off[jj] = run;
        run += loc[r];
    }
    if (tid == 0) s_off[T] = total;
    lds_barrier();
#pragma unroll
    for (int r = 0; r < kW4Max * 128 / kSortT; ++r) {
        const int i = tid + kSortT * r;
        const int k = i < n ? asg[i] : -1;
        if ((unsigned)k < (unsigned)T) {
            const int w4 = i >> 7;
            const uint4 q = bm4[k * W4 + w4];
            const int sh = i & 127;  // bits of this 128-bit word below bit i
            const uint32_t m0 = sh >= 32 ? 0xFFFFFFFFu : (1u << sh) - 1u;
            const uint32_t m1 = sh >= 64 ? 0xFFFFFFFFu : (sh <= 32 ? 0u : (1u << (sh - 32)) - 1u);
            const uint32_t m2 = sh >= 96 ? 0xFFFFFFFFu : (sh <= 64 ? 0u : (1u << (sh - 64)) - 1u);
            const uint32_t m3 = sh <= 96 ? 0u : (1u << (sh - 96)) - 1u;
            const int rank = pre4[k * W4 + w4] + __popc(q.x & m0) + __popc(q.y & m1) +
                             __popc(q.z & m2) + __popc(q.w & m3);
            perm[s_off[k] + rank] = i;
        }
    }
    lds_barrier();
}

// ------------------------------------------------------------ Lloyd update

// New centroids of one event's slots j = tid, tid+256, ... < T: the
// charge-weighted mean of the members perm[s_off[j] .. s_off[j+1]) in that
// (ascending pulse) order, float64, rounded to float32; a zero-weight slot
// keeps its centroid.  Member loads are issued kBatch at a time.
__device__ __forceinline__ void lloyd_slot_means(const LloydArgs& a, int64_t b, int64_t off, int T,
                                                 const int* __restrict__ perm, const int* s_off) {
    for (int j = threadIdx.x; j < T; j += kSortT) {
        double W = 0.0, sx = 0.0, sy = 0.0, sz = 0.0, st = 0.0;
        const int e = s_off[j + 1];
        for (int m0 = s_off[j]; m0 < e; m0 += kBatch) {
            int idx[kBatch];
            float4 x[kBatch];
            float w[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q) idx[q] = m0 + q < e ? perm[m0 + q] : -1;
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                if (idx[q] >= 0) {
                    x[q] = a.coords[off + idx[q]];
                    w[q] = a.charge_col >= 0
                               ? a.features[(off + idx[q]) * (int64_t)a.C + a.charge_col]
                               : 1.0f;
                }
            }
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                if (idx[q] >= 0) {
                    const double wd = (double)w[q];
                    W += wd;
                    sx += wd * (double)x[q].x;
                    sy += wd * (double)x[q].y;
                    sz += wd * (double)x[q].z;
                    st += wd * (double)x[q].w;
                }
            }
        }
        if (W > 0.0)
            a.centroids[b * a.P + j] =
                make_float4((float)(sx / W), (float)(sy / W), (float)(sz / W), (float)(st / W));
    }
}

// lloyd_slot_means from LDS: coordinates rows[i] and weights wts[i] of the
// event's pulses, row n all zero (a batch is padded with it: adding 0.0 * 0.0
// leaves a sum that started at +0.0 unchanged, and the fused multiply-add of
// an exact float64 product rounds once, like the separate add).
__device__ __forceinline__ void lloyd_slot_means_lds(const LloydArgs& a, int64_t b, int n, int T,
                                                     const int* __restrict__ perm,
                                                     const int* s_off,
                                                     const float4* __restrict__ rows,
                                                     const float* __restrict__ wts) {
    for (int j = threadIdx.x; j < T; j += kSortT) {
        double W = 0.0, sx = 0.0, sy = 0.0, sz = 0.0, st = 0.0;
        const int e = s_off[j + 1];
        for (int m0 = s_off[j]; m0 < e; m0 += kBatch) {
            int idx[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q) idx[q] = m0 + q < e ? perm[m0 + q] : n;
            float4 x[kBatch];
            float w[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                x[q] = rows[idx[q]];
                w[q] = wts[idx[q]];
            }
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const double wd = (double)w[q];
                W += wd;
                sx = __builtin_fma(wd, (double)x[q].x, sx);
                sy = __builtin_fma(wd, (double)x[q].y, sy);
                sz = __builtin_fma(wd, (double)x[q].z, sz);
                st = __builtin_fma(wd, (double)x[q].w, st);
            }
        }
        if (W > 0.0)
            a.centroids[b * a.P + j] =
                make_float4((float)(sx / W), (float)(sy / W), (float)(sz / W), (float)(st / W));
    }
}

// One workgroup per event with n > P: every slot's charge-weighted mean of
// its members in ascending pulse order.  An event of up to kLdsPerm pulses
// first copies its coordinates, weights and slots to LDS (dynamic: float4
// rows[kLdsPerm + 1], float wts[kLdsPerm + 1], int slots[kLdsPerm + 1]),
// every load of the copy issued before any is used, and sorts by slot in
// LDS (through bitmaps when n <= 1024, and for n < 2048 through bitmaps kept
// in the rows' unused upper half; else the ballot-match sort); larger events
// sort into device memory and gather their members from it.
constexpr int kLloydBmRows = 2 * kBmW4 * 128;  // events below this size: bitmaps in the rows' upper half
static_assert(2 * kLloydBmRows <= kLdsPerm + 1 && 2 * kLloydBmRows <= kLdsPerm,
              "the upper half of the rows and the prefix table must fit");
__global__ __launch_bounds__(kSortT) void lloyd_update_kernel(LloydArgs a) {
    __shared__ __align__(16) int s_cnt[kSortW * kMaxP];
    __shared__ int s_off[kMaxP + 1];
    __shared__ __align__(16) int s_perm[kLdsPerm];
    extern __shared__ __align__(16) float4 s_rows[];
    const int64_t b = blockIdx.x;
    int64_t off;
    int n;
    event_range(a.offsets, a.N, b, off, n);
    if (n <= a.P) return;
    int T = a.token_count[b];
    T = T > a.P ? a.P : T;
    if (T < 1) return;
    const int tid = threadIdx.x;
    if (n > kLdsPerm) {
        block_sort_by_token(a.assign + off, n, T, a.perm + off, s_cnt, s_off);
        lloyd_slot_means(a, b, off, T, a.perm + off, s_off);
        return;
    }
    float* s_w = reinterpret_cast<float*>(s_rows + kLdsPerm + 1);
    int* s_slot = reinterpret_cast<int*>(s_w + kLdsPerm + 1);
    {
        // all of the event's loads in flight at once (a loop that stored
        // each load before issuing the next would wait a full memory round
        // trip per 256 pulses); indices clamped into the event
        constexpr int R = kLdsPerm / kSortT;
        const int rmax = (n + kSortT - 1) / kSortT;
        float4 x[R];
        float w[R];
        int k[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            x[r] = make_float4(0.f, 0.f, 0.f, 0.f);
            w[r] = 0.0f;
            k[r] = 0;
            if (r < rmax) {
                const int i = min(tid + kSortT * r, n - 1);
                x[r] = a.coords[off + i];
                w[r] = a.charge_col >= 0 ? a.features[(off + i) * (int64_t)a.C + a.charge_col]
                                         : 1.0f;
                k[r] = a.assign[off + i];
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = tid + kSortT * r;
            if (r < rmax && i < n) {
                s_rows[i] = x[r];
                s_w[i] = w[r];
                s_slot[i] = k[r];
            }
        }
    }
    if (tid == 0) {
        s_rows[n] = make_float4(0.f, 0.f, 0.f, 0.f);
        s_w[n] = 0.0f;
    }
    // both sorts start with a barrier before they read the slots
    const int W4 = (n + 127) >> 7;
    if (n <= kBmW4 * 128 && T * W4 <= kLdsPerm / 4) {
        // permutation in s_perm[1024, 2048); prefix table in s_perm[2048,
        // 3072); bitmaps in s_cnt
        int* perm = s_perm + kBmW4 * 128;
        block_sort_bitmap(s_slot, n, T, reinterpret_cast<uint32_t*>(s_cnt),
                          s_perm + 2 * kBmW4 * 128, s_off, perm);
        lloyd_slot_means_lds(a, b, n, T, perm, s_off, s_rows, s_w);
    } else if (n < kLloydBmRows && T * W4 <= kLloydBmRows) {
        // rows 0 .. n (the zero row included) lie below kLloydBmRows, so
        // rows kLloydBmRows .. 2 kLloydBmRows - 1 (16 bytes each) are free for
        // the bitmaps (T * W4 * 16 bytes); permutation in s_perm[0, n),
        // prefix table in s_perm[kLloydBmRows, kLloydBmRows + T * W4)
        block_sort_bitmap<2 * kBmW4>(s_slot, n, T,
                                     reinterpret_cast<uint32_t*>(s_rows + kLloydBmRows),
                                     s_perm + kLloydBmRows, s_off, s_perm);
        lloyd_slot_means_lds(a, b, n, T, s_perm, s_off, s_rows, s_w);
    } else {
        block_sort_by_token(s_slot, n, T, s_perm, s_cnt, s_off);
        lloyd_slot_means_lds(a, b, n, T, s_perm, s_off, s_rows, s_w);
    }
}

// --------------------------------------------------------------------- pool

constexpr int kPoolCols = 8;  // feature columns accumulated per pass

__device__ __forceinline__ void pool_write(const PoolArgs& a, int64_t b, int j, int c0, int nc,
                                           double W, const double* S) {
    float* __restrict__ out = a.pooled + (b * a.P + j) * (int64_t)a.C + c0;
#pragma unroll
    for (int q = 0; q < kPoolCols; ++q)
        if (q < nc) out[q] = W != 0.0 ? (float)(S[q] / W) : 0.0f;
}

// (Weighted) mean of columns [c0, c0+nc) over members given by `member(m)`
// for m in [beg, end), in that order, float64; loads issued kBatch at a time.
template <class Member>
__device__ __forceinline__ void pool_slot_acc(const PoolArgs& a, int64_t off, int beg, int end,
                                              int c0, int nc, Member member, double& W,
                                              double* S) {
    const int C = a.C;
    for (int m0 = beg; m0 < end; m0 += kBatch) {
        int idx[kBatch];
        float w[kBatch];
        float f[kBatch][kPoolCols];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) idx[q] = m0 + q < end ? member(m0 + q) : -1;
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            if (idx[q] >= 0) {
                const float* __restrict__ row = a.features + (off + idx[q]) * (int64_t)C;
                w[q] = a.weight_col >= 0 ? row[a.weight_col] : 1.0f;
#pragma unroll
                for (int c = 0; c < kPoolCols; ++c)
                    if (c < nc) f[q][c] = row[c0 + c];
            }
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            if (idx[q] >= 0) {
                const double wd = (double)w[q];
                W += wd;
#pragma unroll
                for (int c = 0; c < kPoolCols; ++c)
                    if (c < nc) S[c] += wd * (double)f[q][c];
            }
        }
    }
}

template <class Member>
__device__ __forceinline__ void pool_slot(const PoolArgs& a, int64_t off, int beg, int end,
                                          int c0, int nc, Member member, double& W, double* S) {
    W = 0.0;
#pragma unroll
    for (int q = 0; q < kPoolCols; ++q) S[q] = 0.0;
    pool_slot_acc(a, off, beg, end, c0, nc, member, W, S);
}

__device__ __forceinline__ void pool_slots_sorted(const PoolArgs& a, int64_t b, int64_t off,
                                                  int T, const int* __restrict__ perm,
                                                  const int* s_off) {
    const int C = a.C;
    for (int j = threadIdx.x; j < a.P; j += kSortT) {
        const int beg = j < T ? s_off[j] : 0;
        const int end = j < T ? s_off[j + 1] : 0;
        for (int c0 = 0; c0 < C; c0 += kPoolCols) {
            const int nc = min(kPoolCols, C - c0);
            double W, S[kPoolCols];
            pool_slot(a, off, beg, end, c0, nc, [&](int m) { return perm[m]; }, W, S);
            pool_write(a, b, j, c0, nc, W, S);
        }
        if (a.cell_count) a.cell_count[b * a.P + j] = end - beg;
    }
}

// Pooling of an event whose slot j is pulse j alone (j < T): each pulse's
// features through the general formula (w f / w, exact for w != 0).
__device__ __forceinline__ void pool_identity(const PoolArgs& a, int64_t b, int64_t off, int T) {
    const int C = a.C;
    for (int j = threadIdx.x; j < a.P; j += blockDim.x) {
        if (j < T) {
            const float* __restrict__ row = a.features + (off + j) * (int64_t)C;
            float* __restrict__ out = a.pooled + (b * a.P + j) * (int64_t)C;
            const double w = a.weight_col >= 0 ? (double)row[a.weight_col] : 1.0;
            // a group of columns is loaded whole before any is written, so
            // the loads overlap
            constexpr int U = 8;
            for (int c0 = 0; c0 < C; c0 += U) {
                float f[U];
#pragma unroll
                for (int u = 0; u < U; ++u) f[u] = row[min(c0 + u, C - 1)];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (c0 + u < C) out[c0 + u] = w != 0.0 ? (float)((w * (double)f[u]) / w) : 0.0f;
            }
        } else {
            for (int c = 0; c < C; ++c) a.pooled[(b * a.P + j) * (int64_t)C + c] = 0.0f;
        }
        if (a.cell_count) a.cell_count[b * a.P + j] = j < T ? 1 : 0;
    }
}

// ------------------------------ Voronoi pooling by chunks, counting sort

// Orders this wave's LDS accesses before and after it (the wave's LDS
// operations complete in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Stable counting sort of one chunk's pulses by slot, in LDS:
// perm[off_[j] + r] = the r-th pulse (ascending) of the chunk with slot j.
//  1. every wave counts the slots of its contiguous quarter of the chunk
//     with LDS atomics (the order of the counts does not matter);
//  2. an exclusive scan over the slots, then per (wave, slot) the first
//     position of that wave's members of the slot;
//  3. every wave walks its quarter 64 pulses at a time in ascending order:
//     each pulse sets its lane's bit in its wave's 64-bit mask of its slot
//     (an LDS atomic OR), reads the mask back -- the lanes below it with
//     its slot give its rank -- and lands at the slot's cursor plus that
//     rank; the slot's lowest lane then advances the cursor and clears the
//     mask.  Waves touch only their own cursors and masks, and a wave's LDS
//     operations complete in order, so no barrier is needed inside the walk.
//   k: LDS int[len] slots (outside [0, T): left out);  perm: LDS int[len];
//   cnt: LDS int[4 * T];  off_: LDS int[T + 1];  bm: LDS uint64[4 * T], zero
//   on entry and on return.
__device__ __forceinline__ void chunk_sort(const int* k, int len, int T, int* perm, int* cnt,
                                           int* off_, unsigned long long* bm) {
    __shared__ int s_ws[kSortW];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int q = ((len + kSortW - 1) / kSortW + 63) & ~63;  // pulses per wave, whole windows
    const int qb = wave * q, qe = min(len, qb + q);
    int* __restrict__ wc = cnt + wave * T;
    unsigned long long* __restrict__ wm = bm + wave * T;
    for (int i = qb + lane; i < qe; i += 64) {
        const int kk = k[i];
        if ((unsigned)kk < (unsigned)T) atomicAdd(&wc[kk], 1);
    }
    __syncthreads();
    // slot totals and their exclusive scan (thread t: slots t*per ..)
    const int per = (T + kSortT - 1) / kSortT;
    int loc[kMaxP / kSortT];
    int local = 0;
#pragma unroll
    for (int r = 0; r < kMaxP / kSortT; ++r) {
        const int jj = tid * per + r;
        int t = 0;
        if (r < per && jj < T)
#pragma unroll
            for (int w = 0; w < kSortW; ++w) t += cnt[w * T + jj];
        loc[r] = t;
        local += t;
    }
    const int incl = wave_incl_scan(local);
    if (lane == 63) s_ws[wave] = incl;
    __syncthreads();
    int run = incl - local, total = 0;
#pragma unroll
    for (int w = 0; w < kSortW; ++w) {
        const int v = s_ws[w];
        run += w < wave ? v : 0;
        total += v;
    }
#pragma unroll
    for (int r = 0; r < kMaxP / kSortT; ++r) {
        const int jj = tid * per + r;
        if (r < per && jj < T) {
            off_[jj] = run;
            int pos = run;
#pragma unroll
            for (int w = 0; w < kSortW; ++w) {
                const int v = cnt[w * T + jj];
                cnt[w * T + jj] = pos;
                pos += v;
            }
        }
        run += loc[r];
    }
    if (tid == 0) off_[T] = total;
    __syncthreads();
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int t0 = qb; t0 < qe; t0 += 64) {
        const int i = t0 + lane;
        const int kk = i < qe ? k[i] : -1;
        const bool ok = (unsigned)kk < (unsigned)T;
        const int ks = ok ? kk : 0;
        if (ok) atomicOr(&wm[ks], 1ull << lane);
        wave_lds_order();
        const unsigned long long m = wm[ks];
        const int cur = wc[ks];
        wave_lds_order();
        const int rank = __popcll(m & below);
        if (ok) perm[cur + rank] = i;
        if (ok && rank == 0) {
            wc[ks] = cur + __popcll(m);
            wm[ks] = 0ull;
        }
        wave_lds_order();
    }
    __syncthreads();
}

// Columns [c0, c0 + NC) of one slot's (weighted) sums over its members
// perm[mb .. me) (chunk-local pulses, ascending), rows gathered from device
// memory kBatch members at a time; every load of a batch is issued before
// any is used (indices past the slot re-read its last member, unused).
template <int NC>
__device__ __forceinline__ void chunk_slot_gather(const float* __restrict__ rows, int C, int wcol,
                                                  const int* perm, int mb, int me, int c0,
                                                  double& W, double (&S)[NC]) {
    W = 0.0;
#pragma unroll
    for (int q = 0; q < NC; ++q) S[q] = 0.0;
    for (int m0 = mb; m0 < me; m0 += kBatch) {
        int idx[kBatch];
#pragma unroll
        for (int t = 0; t < kBatch; ++t) idx[t] = perm[min(m0 + t, me - 1)];
        float wv[kBatch], fv[kBatch][NC];
#pragma unroll
        for (int t = 0; t < kBatch; ++t) {
            const float* __restrict__ r = rows + (int64_t)idx[t] * C;
            wv[t] = r[wcol >= 0 ? wcol : 0];
#pragma unroll
            for (int q = 0; q < NC; ++q) fv[t][q] = r[c0 + q];
        }
#pragma unroll
        for (int t = 0; t < kBatch; ++t) {
            if (m0 + t < me) {
                const double wd = wcol >= 0 ? (double)wv[t] : 1.0;
                W += wd;
#pragma unroll
                for (int q = 0; q < NC; ++q) S[q] = __builtin_fma(wd, (double)fv[t][q], S[q]);
            }
        }
    }
}

// One column pass of a chunk: every slot's sums, then either the means of a
// one-chunk event (slots j < P, zeros beyond T) or the chunk's record.
template <int NC>
__device__ __forceinline__ void chunk_pass_gather(const PoolArgs& a, int64_t b,
                                                  const float* rows, int T, int c0,
                                                  const int* perm, const int* off_, int part) {
    const int P = a.P;
    const int C = a.C;
    const int C2 = C + 2;
    for (int j = threadIdx.x; j < (part < 0 ? P : T); j += kSortT) {
        const int mb = j < T ? off_[j] : 0, me = j < T ? off_[j + 1] : 0;
        double W, S[NC];
        chunk_slot_gather<NC>(rows, C, a.weight_col, perm, mb, me, c0, W, S);
        if (part < 0) {
            float* __restrict__ out = a.pooled + (b * P + j) * (int64_t)C + c0;
#pragma unroll
            for (int q = 0; q < NC; ++q) out[q] = W != 0.0 ? (float)(S[q] / W) : 0.0f;
            if (c0 == 0 && a.cell_count) a.cell_count[b * P + j] = me - mb;
        } else {
            double* __restrict__ r = a.part + ((size_t)part * P + j) * C2;
            r[0] = W;
#pragma unroll
            for (int q = 0; q < NC; ++q) r[1 + c0 + q] = S[q];
            if (c0 == 0) r[C + 1] = (double)(me - mb);
        }
    }
}

// Voronoi pooling over the chunk list (kPoolChunk pulses per chunk), one
// workgroup per chunk:
//  * an event whose slots are its pulses (n <= P) is pooled pulse by pulse;
//  * otherwise the chunk's slots are copied to LDS and sorted there (stable
//    counting sort, chunk_sort), and thread j sums slot j's members in
//    ascending order with their rows gathered from device memory;
//  * an event of one chunk writes its means; a chunk of a larger event
//    writes its record (weight, every column, member count per slot) for
//    the combine kernel;
//  * an event marked to be summed whole (the caller's bound ruled it out, or
//    malformed offsets left no record space) is sorted and summed by its
//    first chunk's workgroup through device memory.
// Dynamic LDS: int k[kPoolChunk], int perm[kPoolChunk], uint64 bm[4 * P],
// int cnt[4 * P], int off[P + 1].
__global__ __launch_bounds__(kSortT) void pool_chunk_kernel(PoolArgs a) {
    extern __shared__ __align__(16) int s_dyn[];
    const int c = blockIdx.x;
    if (c >= a.header[6]) return;
    const int64_t b = a.chunk_ev[c];
    const int beg = a.chunk_beg[c];
    const int part = a.chunk_part[c];
    int64_t off;
    int n;
    event_range(a.offsets, a.N, b, off, n);
    int T = a.token_count[b];
    T = T < 0 ? 0 : (T > a.P ? a.P : T);
    const int tid = threadIdx.x;
    const int P = a.P;
    const int C = a.C;
    unsigned long long* bm = reinterpret_cast<unsigned long long*>(s_dyn);  // 4 * P
    int* s_k = reinterpret_cast<int*>(bm + kSortW * P);                      // kPoolChunk
    int* perm = s_k + kPoolChunk;                                            // kPoolChunk
    int* cnt = perm + kPoolChunk;                                            // 4 * P
    int* off_ = cnt + kSortW * P;                                            // P + 1
    if (part == -2) {
        if (beg != 0) return;
        for (int q = tid; q < kSortW * P; q += kSortT) cnt[q] = 0;
        __syncthreads();
        block_sort_by_token(a.assign + off, n, T, a.perm + off, cnt, off_);
        pool_slots_sorted(a, b, off, T, a.perm + off, off_);
        return;
    }
    if (part == -1) {
        bool ident = n == T;
        for (int i = tid; ident && i < n; i += kSortT) ident = a.assign[off + i] == i;
        if (__syncthreads_and(ident)) {
            pool_identity(a, b, off, T);
            return;
        }
    }
    const int len = max(0, min(n - beg, kPoolChunk));
    if (len > 0) {
        // the chunk's slots, every load of a thread issued together
        constexpr int R = kPoolChunk / kSortT;
        int v[R];
        const int32_t* __restrict__ ag = a.assign + off + beg;
#pragma unroll
        for (int r = 0; r < R; ++r) v[r] = ag[min(tid + kSortT * r, len - 1)];
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (tid + kSortT * r < len) s_k[tid + kSortT * r] = v[r];
    }
    for (int q = tid; q < kSortW * T; q += kSortT) {
        cnt[q] = 0;
        bm[q] = 0ull;
    }
    __syncthreads();
    chunk_sort(s_k, len, T, perm, cnt, off_, bm);
    const float* __restrict__ rows = a.features + (off + beg) * (int64_t)C;
    for (int c0 = 0; c0 < C; c0 += kPoolCols) {
        switch (min(kPoolCols, C - c0)) {
#define FPSTOK_GATHER_PASS(NC) \
    case NC: chunk_pass_gather<NC>(a, b, rows, T, c0, perm, off_, part); break;
            FPSTOK_GATHER_PASS(1)
            FPSTOK_GATHER_PASS(2)
            FPSTOK_GATHER_PASS(3)
            FPSTOK_GATHER_PASS(4)
            FPSTOK_GATHER_PASS(5)
            FPSTOK_GATHER_PASS(6)
            FPSTOK_GATHER_PASS(7)
            default: FPSTOK_GATHER_PASS(8)
#undef FPSTOK_GATHER_PASS
        }
    }
}

// --------------- Voronoi pooling by chunks, rows sorted by slot into LDS

constexpr int kSrtT = 512;               // threads of the sorting pooling kernel
constexpr int kSrtW = kSrtT / 64;        // its waves
constexpr int kSrtR = kPoolChunk / kSrtT;  // pulses per thread (8)
constexpr int kSrtMaxP = 256;            // slots it handles (one per thread of the first waves)
constexpr int kSrtMaxC = 6;              // widest rows it handles
static_assert(kSrtR * kSrtT == kPoolChunk, "one pulse per thread and window");

// Voronoi pooling over the chunk list (kPoolChunk pulses per chunk) for P
// <= 256 and rows of at most 6 columns: one workgroup of 512 threads per
// compute unit takes one chunk per round of gridDim chunks, in serpentine
// order (round k: workgroup g takes chunk k gridDim + g for even k and
// k gridDim + gridDim - 1 - g for odd k; the planner lists the chunks
// longest first, so the rounds even out the workgroups' loads) and, while it
// pools one, has the next one's slots and rows loading into registers.  A
// chunk of len pulses is cut into R = ceil(len / 512) 64-pulse windows per
// wave: wave w holds pulses 64 R w .. 64 R (w + 1) - 1 (lane l of window r:
// pulse 64 R w + 64 r + l), so the windows are in pulse order wave after
// wave and a short chunk costs only the windows it fills.  A chunk:
//  1. every pulse counts its slot per wave (LDS atomics; order irrelevant);
//  2. per slot, an exclusive scan gives the slot's first row; per (wave,
//     slot), the first row of that wave's members;
//  3. every wave ranks each window's pulses among their equal-slot lanes
//     (each lane sets its bit in its wave's 64-bit mask of its slot, an LDS
//     atomic OR, and reads the mask back: the lanes below it in the mask
//     give its rank), writes each row to LDS at its wave's cursor plus that
//     rank, and the slot's lowest lane advances the cursor and clears the
//     mask: the rows of every slot land in ascending pulse order, one after
//     the other;
//  4. thread j adds slot j's rows -- contiguous in LDS -- in that order into
//     float64 sums: each slot's chunk sum is one ascending sequence, the
//     oracle's operations in the oracle's order.
// Then an event of one chunk writes its means (0 beyond T; events whose slots
// are their pulses, n <= P, are pooled pulse by pulse), a chunk of a larger
// event writes its record for the combine kernel, and an event marked to be
// summed whole (the caller's bound ruled it out, or malformed offsets left
// no record space) is taken by its first chunk's workgroup sub-chunk after
// sub-chunk, one ascending sum.  Every barrier orders LDS only, so the next
// chunk's loads stay in flight across the chunk in hand, and the kernel has
// no fence (the kernel boundary publishes the records).  The chunks'
// descriptions (event, range, record, token count) are read 64 at a time
// into LDS, so their chain of dependent loads is paid once per 64 chunks.
// Dynamic LDS: float rows[kPoolChunk * NC], float zero[kSrtZero] (a zero
// row), int cnt[kSrtW * P], int off[P + 1], uint64 bm[kSrtW * P] (zero
// between chunks).
constexpr int kSrtMeta = 64;  // chunk descriptions read at a time
constexpr int kSrtZero = 8;   // floats of the zero row (>= kSrtMaxC; keeps cnt 16-byte aligned)
static_assert(kSrtZero >= kSrtMaxC && kSrtZero % 4 == 0, "zero row");
// 64-pulse windows per wave for a chunk of len pulses (0 for an empty one)
// on kW waves
template <int kW = kSrtW>
__device__ __forceinline__ int srt_windows(int len) {
    return __builtin_amdgcn_readfirstlane((max(len, 0) + 64 * kW - 1) / (64 * kW));
}
// Steps 1-3 above for one sub-chunk of at most 64 kW kR pulses on a
// workgroup of kW waves (this thread's pulses 64 R wave + 64 r + lane,
// r < R: slots k[r], rows f[r]): the rows land in LDS sorted by slot, slot
// j's at off_[j] .. off_[j + 1] (T <= 64 kW slots).  cnt: LDS int[kW T],
// bm: LDS uint64[kW T], zero on entry and on return; s_ws: LDS int[kW].
// Ends with a workgroup barrier; k and f are not needed afterwards.
template <int NC, int kW = kSrtW, int kR = kSrtR>
__device__ __forceinline__ void sorted_place(const int (&k)[kR], const float (&f)[kR][NC],
                                             int len, int T, float* s_rows, int* cnt, int* off_,
                                             int* s_ws, unsigned long long* bm) {
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int R = srt_windows<kW>(len);
    const int w0 = 64 * R * wave;  // this wave's first pulse
    // 1. counts per (wave, slot)
    for (int q = tid; q < kW * T; q += 64 * kW) cnt[q] = 0;
    lds_barrier();
    int* __restrict__ wc = cnt + wave * T;
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        const int i = w0 + 64 * r + lane;
        if (r < R && i < len && (unsigned)k[r] < (unsigned)T) atomicAdd(&wc[k[r]], 1);
    }
    lds_barrier();
    // 2. slot offsets and (wave, slot) cursors (threads j < T)
    {
        const int j = tid;
        int tot = 0;
        if (j < T)
#pragma unroll
            for (int w = 0; w < kW; ++w) tot += cnt[w * T + j];
        const int incl = wave_incl_scan(tot);
        if (lane == 63) s_ws[wave] = incl;
        lds_barrier();
        int run = incl - tot;
        for (int w = 0; w < wave; ++w) run += s_ws[w];
        if (j < T) {
            off_[j] = run;
            int pos = run;
#pragma unroll
            for (int w = 0; w < kW; ++w) {
                const int v = cnt[w * T + j];
                cnt[w * T + j] = pos;
                pos += v;
            }
        }
        if (j == 0) {
            int total = 0;
            for (int w = 0; w < kW; ++w) total += s_ws[w];
            off_[T] = total;
        }
    }
    lds_barrier();
    // 3. rows to their sorted places, window after window per wave
    unsigned long long* __restrict__ wm = bm + wave * T;
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        if (r >= R) break;  // R is uniform: the whole workgroup leaves together
        const int i = w0 + 64 * r + lane;
        const bool ok = i < len && (unsigned)k[r] < (unsigned)T;
        const int kk = ok ? k[r] : 0;
        if (ok) atomicOr(&wm[kk], 1ull << lane);
        wave_lds_order();
        const unsigned long long m = wm[kk];
        const int cur = wc[kk];
        wave_lds_order();
        const int rank = __popcll(m & below);
        if (ok) {
            float* __restrict__ dst = s_rows + (cur + rank) * NC;
#pragma unroll
            for (int q = 0; q < NC; ++q) dst[q] = f[r][q];
            if (rank == 0) {
                wc[kk] = cur + __popcll(m);
                wm[kk] = 0ull;
            }
        }
        wave_lds_order();
    }
    lds_barrier();
}

// Step 4: thread j < T adds slot j's sorted rows, in order, into its
// float64 sums (which carry over from earlier sub-chunks).  Ends with a
// barrier that orders LDS only.
template <int NC>
__device__ __forceinline__ void sorted_sums(int T, int wcol, const float* s_rows,
                                            const float* zrow, const int* off_, double& W,
                                            double (&S)[NC], int& count) {
    const int tid = threadIdx.x;
    if (tid < T) {
        const int mb = off_[tid], me = off_[tid + 1];
        // four members' rows read together, then added one after the other,
        // with no per-member branch: a member past the slot reads the zero
        // row that follows the rows, so it adds weight +0 and products +0.
        // Those leave every sum as it was: the sums start at +0, and under
        // rounding to nearest a sum that starts at +0 never becomes -0.
        // the weight as bits: the row's weight column, or 1.0 for a member
        // and 0 past the slot when there is none (no branch on either)
        const bool weighted = wcol >= 0 && wcol < NC;
        const int wc = weighted ? wcol : 0;
        const int wkeep = weighted ? -1 : 0;
        const int wone = weighted ? 0 : 0x3f800000;
        constexpr int U = 4;
        for (int m0 = mb; m0 < me; m0 += U) {
            float fv[U][NC], wv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool ok = m0 + u < me;
                const float* __restrict__ rw = ok ? s_rows + (m0 + u) * NC : zrow;
#pragma unroll
                for (int q = 0; q < NC; ++q) fv[u][q] = rw[q];
                wv[u] = __int_as_float((__float_as_int(rw[wc]) & wkeep) | (ok ? wone : 0));
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const double wd = (double)wv[u];
                W += wd;
#pragma unroll
                for (int q = 0; q < NC; ++q) S[q] = __builtin_fma(wd, (double)fv[u][q], S[q]);
            }
        }
        count += me - mb;
    }
    lds_barrier();
}

template <int NC>
__global__ __launch_bounds__(kSrtT) void pool_sorted_kernel(PoolArgs a) {
    extern __shared__ __align__(16) float s_srt[];
    float* s_rows = s_srt;
    __shared__ int s_ws[kSrtW];
    __shared__ int s_vote[kSrtW];
    __shared__ int s_mb[kSrtMeta], s_mbeg[kSrtMeta], s_mpart[kSrtMeta], s_mn[kSrtMeta],
        s_mT[kSrtMeta];
    __shared__ int64_t s_moff[kSrtMeta];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int P = a.P;
    const int C = NC;
    const int wcol = a.weight_col;
    int* cnt = reinterpret_cast<int*>(s_rows + kPoolChunk * NC + kSrtZero);  // [kSrtW][P]
    int* off_ = cnt + kSrtW * P;                                             // [P + 1]
    unsigned long long* bm = reinterpret_cast<unsigned long long*>(
        off_ + ((P + 2) & ~1));                                              // [kSrtW][P]
    for (int q = tid; q < kSrtW * P; q += kSrtT) bm[q] = 0ull;
    const float* zrow = s_rows + kPoolChunk * NC;
    if (tid < kSrtZero) s_rows[kPoolChunk * NC + tid] = 0.0f;
    const int nchunks = a.header[6];
    const int G = gridDim.x;
    // this workgroup's chunk of round i (serpentine order); increasing in i
    auto chunk_of = [&](int i) {
        return i * G + ((i & 1) ? G - 1 - (int)blockIdx.x : (int)blockIdx.x);
    };
    // descriptions of this workgroup's chunks of rounds i0 .. i0 + 63, read
    // by wave 0; the callers put a barrier after
    auto fill_meta = [&](int i0) {
        if (wave == 0) {
            const int c = chunk_of(i0 + lane);
            int b = 0, beg = 0, part = -1, n = 0, T = 0;
            int64_t off = 0;
            if (c < nchunks) {
                b = a.chunk_ev[c];
                beg = a.chunk_beg[c];
                part = a.chunk_part[c];
                event_range(a.offsets, a.N, b, off, n);
                T = a.token_count[b];
            }
            s_mb[lane] = b;
            s_mbeg[lane] = beg;
            s_mpart[lane] = part;
            s_mn[lane] = n;
            s_mT[lane] = T < 0 ? 0 : (T > P ? P : T);
            s_moff[lane] = off;
        }
    };
    // a sub-chunk's pulses of this thread (64 R wave + 64 r + lane, r < R)
    // into k, f, indices clamped into it so that every load is issued
    // together (windows r >= R load its last pulse, which nothing reads); an
    // empty sub-chunk loads nothing (its first row may lie past the input)
    int k[kSrtR];
    float f[kSrtR][NC];
    auto load = [&](int64_t off, int beg, int len) {
        // the same for every thread: said so, the test below is a scalar
        // branch, and no register of the loads has to be merged (and waited
        // for) where the two ways join
        len = __builtin_amdgcn_readfirstlane(len);
        beg = __builtin_amdgcn_readfirstlane(beg);
        off = ((int64_t)__builtin_amdgcn_readfirstlane((int)(off >> 32)) << 32) |
              (uint32_t)__builtin_amdgcn_readfirstlane((int)off);
        if (len <= 0) {
#pragma unroll
            for (int r = 0; r < kSrtR; ++r) {
                k[r] = -1;
#pragma unroll
                for (int q = 0; q < NC; ++q) f[r][q] = 0.0f;
            }
            return;
        }
        const int32_t* __restrict__ ag = a.assign + off + beg;
        const float* __restrict__ fg = a.features + (off + beg) * (int64_t)C;
        const int R = srt_windows(len);
#pragma unroll
        for (int r = 0; r < kSrtR; ++r) {
            const int i = r < R ? min(64 * R * wave + 64 * r + lane, len - 1) : len - 1;
            k[r] = ag[i];
#pragma unroll
            for (int q = 0; q < NC; ++q) f[r][q] = fg[(int64_t)i * C + q];
        }
    };
    // the data of local chunk i (description in LDS slot i - m0)
    auto load_local = [&](int i, int m0) {
        const int m = i - m0;
        const int n = s_mn[m], beg = s_mbeg[m];
        load(s_moff[m], beg, max(0, min(n - beg, kPoolChunk)));
    };
    int m0 = 0;  // local index of the first description in LDS
    fill_meta(0);
    lds_barrier();  // descriptions and cleared masks
    if (chunk_of(0) < nchunks) load_local(0, 0);
    for (int i = 0; chunk_of(i) < nchunks; ++i) {
        const int m = i - m0;
        const int64_t b = s_mb[m];
        const int beg = s_mbeg[m];
        const int part = s_mpart[m];
        const int64_t off = s_moff[m];
        const int n = s_mn[m];
        const int T = s_mT[m];
        const int len = max(0, min(n - beg, kPoolChunk));
        const bool more = chunk_of(i + 1) < nchunks;
        // the next chunk's description, read into LDS here when it is past
        // the ones held (every thread has read chunk i's above)
        if (more && i + 1 - m0 >= kSrtMeta) {
            lds_barrier();
            m0 = i + 1;
            fill_meta(m0);
            lds_barrier();
        }
        if (part == -2 && beg != 0) {
            // summed whole by the event's first chunk
            if (more) load_local(i + 1, m0);
            continue;
        }
        if (part == -1) {
            bool ident = n == T;
            const int R = srt_windows(len);
#pragma unroll
            for (int r = 0; r < kSrtR; ++r) {
                const int ii = 64 * R * wave + 64 * r + lane;
                ident = ident && (r >= R || ii >= len || k[r] == ii);
            }
            const bool wave_ident = ballot(!ident) == 0;
            if (lane == 0) s_vote[wave] = wave_ident ? 1 : 0;
            lds_barrier();
            int all = 1;
#pragma unroll
            for (int w = 0; w < kSrtW; ++w) all &= s_vote[w];
            lds_barrier();  // every wave has read the votes
            if (all) {
                if (more) load_local(i + 1, m0);
                pool_identity(a, b, off, T);
                continue;
            }
        }
        double W = 0.0, S[NC];
#pragma unroll
        for (int q = 0; q < NC; ++q) S[q] = 0.0;
        int count = 0;
        sorted_place<NC>(k, f, len, T, s_rows, cnt, off_, s_ws, bm);
        if (part == -2) {
            // the rest of an event summed whole, sub-chunk after sub-chunk
            // (one ascending sum)
            for (int sb = kPoolChunk; sb < n; sb += kPoolChunk) {
                sorted_sums<NC>(T, wcol, s_rows, zrow, off_, W, S, count);
                const int sl = min(n - sb, kPoolChunk);
                load(off, sb, sl);
                sorted_place<NC>(k, f, sl, T, s_rows, cnt, off_, s_ws, bm);
            }
        }
        // the rows are in LDS: the next chunk's loads go out now, behind the
        // sums and the outputs
        if (more) load_local(i + 1, m0);
        sorted_sums<NC>(T, wcol, s_rows, zrow, off_, W, S, count);
        const int j = tid;
        if (part < 0) {
            if (j < P) {
                float* __restrict__ out = a.pooled + (b * P + j) * (int64_t)C;
#pragma unroll
                for (int q = 0; q < NC; ++q)
                    out[q] = j < T && W != 0.0 ? (float)(S[q] / W) : 0.0f;
                if (a.cell_count) a.cell_count[b * P + j] = j < T ? count : 0;
            }
        } else if (j < T) {
            // this chunk's record for the combine kernel
            constexpr int C2 = NC + 2;
            double* __restrict__ rr = a.part + ((size_t)part * P + j) * C2;
            rr[0] = W;
#pragma unroll
            for (int q = 0; q < NC; ++q) rr[1 + q] = S[q];
            rr[NC + 1] = (double)count;
        }
    }
}

// Means of the events of more than one chunk from their chunks'
// records: block (event m, slot group) with threads (field f, slot js);
// field 0 is the weight, 1..C the columns, C+1 the member count; every
// thread adds its value over the K records in chunk order, kCombineDepth loads in
// flight.
constexpr int kCombineDepth = 16;  // records read together
__global__ __launch_bounds__(256) void pool_combine_kernel(PoolArgs a) {
    __shared__ double s_W[256];
    const int m = blockIdx.x;
    if (m >= a.header[4]) return;
    const int b = a.big_ev[m];
    if (b < 0) return;
    const int p0 = a.big_ev[a.B + m];
    int64_t off;
    int n;
    event_range(a.offsets, a.N, b, off, n);
    const int K = (n + kPoolChunk - 1) / kPoolChunk;
    int T = a.token_count[b];
    T = T < 0 ? 0 : (T > a.P ? a.P : T);
    const int P = a.P;
    const int C = a.C;
    const int C2 = C + 2;
    const int f = threadIdx.x;
    const int js = threadIdx.y;
    const int j = blockIdx.y * blockDim.y + js;
    double t = 0.0;
    if (j < T) {
        const double* __restrict__ r = a.part + ((size_t)p0 * P + j) * C2 + f;
        const size_t stride = (size_t)P * C2;
        for (int k0 = 0; k0 < K; k0 += kCombineDepth) {
            double v[kCombineDepth];
#pragma unroll
            for (int u = 0; u < kCombineDepth; ++u)
                v[u] = k0 + u < K ? r[(size_t)(k0 + u) * stride] : 0.0;
#pragma unroll
            for (int u = 0; u < kCombineDepth; ++u)
                if (k0 + u < K) t += v[u];
        }
    }
    if (f == 0) s_W[js] = t;
    __syncthreads();
    if (j < P) {
        if (f >= 1 && f <= C) {
            const double W = s_W[js];
            a.pooled[((int64_t)b * P + j) * C + f - 1] = j < T && W != 0.0 ? (float)(t / W) : 0.0f;
        } else if (f == C + 1 && a.cell_count) {
            a.cell_count[(int64_t)b * P + j] = j < T ? (int)t : 0;
        }
    }
}

// kNN pooling, one workgroup per event: every slot's list entries that are
// valid pulse indices, in list order.
__global__ __launch_bounds__(kSortT) void pool_knn_kernel(PoolArgs a) {
    const int64_t b = blockIdx.x;
    int64_t off;
    int n;
    event_range(a.offsets, a.N, b, off, n);
    int T = a.token_count[b];
    T = T < 0 ? 0 : (T > a.P ? a.P : T);
    const int C = a.C;
    const int k = a.k;
    for (int j = threadIdx.x; j < a.P; j += kSortT) {
        const int32_t* __restrict__ lst = a.knn_idx + (b * a.P + j) * (int64_t)k;
        const int len = j < T ? k : 0;
        auto member = [&](int e) {
            const int i = lst[e];
            return i < n ? i : -1;
        };
        for (int c0 = 0; c0 < C; c0 += kPoolCols) {
            const int nc = min(kPoolCols, C - c0);
            double W, S[kPoolCols];
            pool_slot(a, off, 0, len, c0, nc, member, W, S);
            pool_write(a, b, j, c0, nc, W, S);
        }
        if (a.cell_count) {
            int count = 0;
            for (int e = 0; e < len; ++e) count += member(e) >= 0 ? 1 : 0;
            a.cell_count[b * a.P + j] = count;
        }
    }
}

// ------------------------------------------- fused FPS + Voronoi pooling

constexpr int kFusedR = 4;                        // 64-pulse windows per wave and sub-chunk
constexpr int kFusedSub = 64 * kFpsW * kFusedR;  // pulses per sub-chunk (1024)
static_assert(kFusedSub * kSrtMaxC <= kStage, "a sub-chunk's rows fit the staging area");
static_assert((sizeof(unsigned long long) + sizeof(int)) * kFpsW * kSrtMaxP + 8 * sizeof(float) <=
                  sizeof(int) * kFpsCap,
              "masks, counts and the zero row fit s_perm");

// Pooling of the cnt pulses one workgroup holds (an event, or a gang's
// shard) for P <= 256 slots and NC <= 6 columns, without gathers: the pulses'
// rows (global rows row0 + i, read whole and in order) and slots (slots[i],
// LDS) go through sub-chunks of kFusedSub pulses, each counted and placed into
// LDS sorted by slot (the standalone pooling's placement, on kFpsW waves) and
// added by its slot's thread into float64 sums that carry over from one
// sub-chunk to the next: every slot's sum is one chain in ascending pulse
// order, the oracle's.  Thread j < T ends with slot j's weight W, sums S and
// member count.  rows: LDS float[kFusedSub * NC]; bm: LDS uint64[kFpsW T] and
// cw: LDS int[kFpsW T] (cleared here); zrow: LDS float[8] (zeroed here);
// off_: LDS int[T + 1]; s_ws: LDS int[kFpsW].
template <int NC>
__device__ __forceinline__ void fused_sorted_sums(const PoolArgs& pa, int64_t row0,
                                                  const int* slots, int cnt, int T, float* rows,
                                                  unsigned long long* bm, int* cw, float* zrow,
                                                  int* off_, int* s_ws, double& W,
                                                  double (&S)[NC], int& count) {
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    cnt = __builtin_amdgcn_readfirstlane(cnt);
    for (int q = tid; q < kFpsW * T; q += kFpsT) bm[q] = 0ull;  // ordered by the placement's barriers
    if (tid < 8) zrow[tid] = 0.0f;
    W = 0.0;
#pragma unroll
    for (int q = 0; q < NC; ++q) S[q] = 0.0;
    count = 0;
    int k[kFusedR];
    float f[kFusedR][NC];
    // a sub-chunk's pulses of this thread (64 R wave + 64 r + lane, r < R),
    // every load issued together (windows r >= R load the last pulse, which
    // nothing reads)
    auto load = [&](int sb) {
        const int len = __builtin_amdgcn_readfirstlane(min(kFusedSub, cnt - sb));
        const int R = srt_windows<kFpsW>(len);
        const float* __restrict__ fg = pa.features + (row0 + sb) * (int64_t)NC;
#pragma unroll
        for (int r = 0; r < kFusedR; ++r) {
            const int i = r < R ? min(64 * R * wave + 64 * r + lane, len - 1) : len - 1;
            k[r] = slots[sb + i];
#pragma unroll
            for (int q = 0; q < NC; ++q) f[r][q] = fg[(int64_t)i * NC + q];
        }
    };
    if (cnt > 0) load(0);
    for (int sb = 0; sb < cnt; sb += kFusedSub) {
        const int len = __builtin_amdgcn_readfirstlane(min(kFusedSub, cnt - sb));
        sorted_place<NC, kFpsW, kFusedR>(k, f, len, T, rows, cw, off_, s_ws, bm);
        // the rows are in LDS: the next sub-chunk's loads go out behind the sums
        if (sb + kFusedSub < cnt) load(sb + kFusedSub);
        sorted_sums<NC>(T, pa.weight_col, rows, zrow, off_, W, S, count);
    }
}

// fused_sorted_sums for one work item, then its outputs: a single-workgroup
// event's means and member counts, or a gang shard's record of float64
// partial sums (weight, then the columns) and member counts.
template <int NC>
__device__ __forceinline__ void fused_sorted_item(const SampleArgs& a, const PoolArgs& pa,
                                                  const ItemInfo& it, int P, const int* slots,
                                                  float* rows, int* s_perm, int* s_off,
                                                  int* s_ws, bool gang) {
    unsigned long long* bm = reinterpret_cast<unsigned long long*>(s_perm);
    int* cw = s_perm + 2 * kFpsW * P;
    float* zrow = reinterpret_cast<float*>(cw + kFpsW * P);
    double W, S[NC];
    int count;
    fused_sorted_sums<NC>(pa, it.off + it.lo, slots, it.cnt, P, rows, bm, cw, zrow, s_off, s_ws,
                          W, S, count);
    const int j = threadIdx.x;
    if (j >= P) return;
    if (!gang) {
        float* __restrict__ out = pa.pooled + (it.b * P + j) * (int64_t)NC;
#pragma unroll
        for (int q = 0; q < NC; ++q) out[q] = W != 0.0 ? (float)(S[q] / W) : 0.0f;
        if (pa.cell_count) pa.cell_count[it.b * P + j] = count;
    } else {
        constexpr int C1 = NC + 1;
        double* __restrict__ pj = a.gang_part + ((size_t)(it.item0 + it.g) * P + j) * C1;
        pj[0] = W;
#pragma unroll
        for (int q = 0; q < NC; ++q) pj[1 + q] = S[q];
        a.shard_cells[(size_t)(it.item0 + it.g) * (P + 1) + j] = count;
    }
}

// Slot j's (weighted) mean of columns c0 .. c0+NC-1 from LDS rows, members
// perm[beg .. end) in that order, kBatch at a time.  A batch is padded with
// row n, which is all zero: adding 0.0 * 0.0 leaves a sum that started at
// +0.0 unchanged, so the result is the same float64 sequence as
// pool_slot_acc's.  The products of two floats are exact in float64, so the
// fused multiply-add rounds once, like the separate add.
template <int NC>
__device__ __forceinline__ void pool_lds_cols(const PoolArgs& a, int64_t b, int j, int beg,
                                              int end, int n, int c0,
                                              const int* __restrict__ perm,
                                              const float* __restrict__ rows) {
    const int C = a.C;
    const int wcol = a.weight_col;
    double W = 0.0, S[NC];
#pragma unroll
    for (int q = 0; q < NC; ++q) S[q] = 0.0;
    for (int m0 = beg; m0 < end; m0 += kBatch) {
        int idx[kBatch];
#pragma unroll
        for (int t = 0; t < kBatch; ++t) idx[t] = m0 + t < end ? perm[m0 + t] : n;
        float wv[kBatch], fv[kBatch][NC];
#pragma unroll
        for (int t = 0; t < kBatch; ++t) {
            const float* __restrict__ row = rows + idx[t] * C;
            wv[t] = wcol >= 0 ? row[wcol] : (idx[t] < n ? 1.0f : 0.0f);
#pragma unroll
            for (int q = 0; q < NC; ++q) fv[t][q] = row[c0 + q];
        }
#pragma unroll
        for (int t = 0; t < kBatch; ++t) {
            const double wd = (double)wv[t];
            W += wd;
#pragma unroll
            for (int q = 0; q < NC; ++q) S[q] = __builtin_fma(wd, (double)fv[t][q], S[q]);
        }
    }
    float* __restrict__ out = a.pooled + (b * a.P + j) * (int64_t)C + c0;
#pragma unroll
    for (int q = 0; q < NC; ++q) out[q] = W != 0.0 ? (float)(S[q] / W) : 0.0f;
}

// Pooling of a single-workgroup event of n pulses whose members are sorted
// by slot in LDS (perm, s_off) and whose feature rows are staged in LDS
// (rows[i * C + c], followed by a zero row): every slot's (weighted) mean
// in ascending member order, float64, from LDS instead of device memory.
// With fewer slots than threads the columns are split into G groups, one
// thread per (slot, group), so that every wave works (each column's sum is
// the same sequence either way).
__device__ __forceinline__ void pool_slots_lds(const PoolArgs& a, int64_t b, int n,
                                               const int* __restrict__ perm, const int* s_off,
                                               const float* __restrict__ rows) {
    const int P = a.P;
    const int C = a.C;
    const int G = max(1, min(C, kFpsT / P));
    const int cpg = (C + G - 1) / G;  // columns per group
    for (int t = threadIdx.x; t < P * G; t += kFpsT) {
        const int j = t % P;
        const int g = t / P;
        const int beg = s_off[j], end = s_off[j + 1];
        const int cend = min(C, (g + 1) * cpg);
        for (int c0 = g * cpg; c0 < cend; c0 += kPoolCols) {
            switch (min(kPoolCols, cend - c0)) {
                case 1: pool_lds_cols<1>(a, b, j, beg, end, n, c0, perm, rows); break;
                case 2: pool_lds_cols<2>(a, b, j, beg, end, n, c0, perm, rows); break;
                case 3: pool_lds_cols<3>(a, b, j, beg, end, n, c0, perm, rows); break;
                case 4: pool_lds_cols<4>(a, b, j, beg, end, n, c0, perm, rows); break;
                case 5: pool_lds_cols<5>(a, b, j, beg, end, n, c0, perm, rows); break;
                case 6: pool_lds_cols<6>(a, b, j, beg, end, n, c0, perm, rows); break;
                case 7: pool_lds_cols<7>(a, b, j, beg, end, n, c0, perm, rows); break;
                default: pool_lds_cols<8>(a, b, j, beg, end, n, c0, perm, rows); break;
            }
        }
        if (g == 0 && a.cell_count) a.cell_count[b * P + j] = end - beg;
    }
}

// Tokenizer in one launch for Voronoi mode without Lloyd: every workgroup
// claims a work item, runs FPS (or pass-through) and then pools its event
// while other workgroups are still sampling.
//  * pass-through: each pulse pooled on its own;
//  * one workgroup: the slots it just computed are sorted in LDS (stable, so
//    each slot's members stay in ascending order) and pooled;
//  * a gang: every shard sorts its own pulses, publishes float64 partial
//    sums (weight and every column) and member counts per slot, raises a
//    tagged flag, waits for all shards, and then finishes the slots j = g,
//    g+G, ... by adding the shards' partials in shard order (each partial in
//    ascending pulse order: only the grouping at shard boundaries differs
//    from one ascending sum);
//  * streaming (beyond gang size): a workgroup-wide sort in device memory.
// Dynamic LDS: s_perm[kFpsCap] (during FPS: the FpsLds of a single-workgroup
// event), s_asg[kFpsCap], s_cnt[kSortW*P], s_off[P+1].
//
// Two instantiations: kDirect (every workgroup takes the event of its own
// index; no gang code at all, so the common small-event kernel's code and
// registers do not depend on the gang path) and the work-list kernel.
template <bool kDirect>
__global__ __launch_bounds__(kFpsT) void tokenize_kernel(SampleArgs a, PoolArgs pa) {
    __shared__ int s_item;
    __shared__ FpsSlot s_slots[2][kFpsW];
    __shared__ int s_sel[FPSTOK_MAX_SLOTS];
    extern __shared__ __align__(16) int s_dyn[];
    // single events keep their FPS state inside s_perm; gangs spill into
    // s_asg, which fps_gang writes only after a final barrier
    static_assert(sizeof(SingleLds) <= sizeof(int) * kFpsCap, "SingleLds must fit in s_perm");
    static_assert(sizeof(GangLds) <= sizeof(int) * 2 * kFpsCap, "GangLds must fit in s_perm+s_asg");
    const int P = a.P;
    int* s_perm = s_dyn;
    int* s_asg = s_perm + kFpsCap;
    int* s_cnt = s_asg + kFpsCap;
    int* s_off = s_cnt + kSortW * P;
    GangLds& s_gang = *reinterpret_cast<GangLds*>(s_perm);
    float* s_feat = reinterpret_cast<float*>(s_off + P + 1);
    // in direct mode no planner clears the device error word (nothing in
    // this mode can set it)
    if (kDirect && blockIdx.x == 0 && threadIdx.x == 0) a.header[3] = 0;
    const ItemInfo it = sample_item<kDirect>(a, &s_item, s_slots, s_gang, s_sel, s_asg, pa.features,
                                             pa.C, pa.stage_cap, s_feat);
    if (it.b < 0) return;
    const int64_t b = it.b;
    const int64_t off = it.off;
    const int tid = threadIdx.x;
    const int C = pa.C;
    if (it.kind == 0) {
        pool_identity(pa, b, off, it.n);
        return;
    }
    if (it.kind == 3) {
        __syncthreads();
        block_sort_by_token(a.assign + off, it.n, P, pa.perm + off, s_cnt, s_off);
        pool_slots_sorted(pa, b, off, P, pa.perm + off, s_off);
        return;
    }
    lds_barrier();
    if (it.kind == 1 && it.deferred) {
        // small event, rows in LDS: the selection's indices now and its
        // coordinates' loads in flight across the sort and pooling (whose
        // barriers order LDS only); bitmap sort into s_asg[1024 ..), pooling
        // from LDS (s_asg holds at most 1024 slots here; P <= 512)
        const int j0 = tid, j1 = tid + kFpsT;
        const int s0 = j0 < P ? s_sel[j0] : 0;
        const int s1 = j1 < P ? s_sel[j1] : 0;
        if (j0 < P) a.centroid_idx[b * P + j0] = s0;
        if (j1 < P) a.centroid_idx[b * P + j1] = s1;
        const float4 c0 = a.coords[off + s0];
        const float4 c1 = a.coords[off + s1];
        int* perm = s_asg + kBmW4 * 128;
        block_sort_bitmap(s_asg, it.n, P, reinterpret_cast<uint32_t*>(s_perm),
                          s_asg + 2 * kBmW4 * 128, s_off, perm);
        pool_slots_lds(pa, b, it.n, perm, s_off, s_feat);
        if (j0 < P) a.centroids[b * P + j0] = c0;
        if (j1 < P) a.centroids[b * P + j1] = c1;
        return;
    }
    const int C1 = C + 1;
    if (P <= kSrtMaxP && C <= kSrtMaxC && pa.stage_cap >= kFusedSub * C) {
        // sub-chunks sorted into LDS: rows in the staging area, masks, counts
        // and the zero row in s_perm (free after FPS), the per-wave totals in
        // s_slots (used only by the streaming FPS)
        int* sws = reinterpret_cast<int*>(s_slots);
        const bool gang = !kDirect && it.kind == 2;
        switch (C) {
            case 1: fused_sorted_item<1>(a, pa, it, P, s_asg, s_feat, s_perm, s_off, sws, gang); break;
            case 2: fused_sorted_item<2>(a, pa, it, P, s_asg, s_feat, s_perm, s_off, sws, gang); break;
            case 3: fused_sorted_item<3>(a, pa, it, P, s_asg, s_feat, s_perm, s_off, sws, gang); break;
            case 4: fused_sorted_item<4>(a, pa, it, P, s_asg, s_feat, s_perm, s_off, sws, gang); break;
            case 5: fused_sorted_item<5>(a, pa, it, P, s_asg, s_feat, s_perm, s_off, sws, gang); break;
            default: fused_sorted_item<6>(a, pa, it, P, s_asg, s_feat, s_perm, s_off, sws, gang); break;
        }
        if (kDirect || !gang) return;
    } else {
        // the shard's pulses sorted by slot: in s_asg itself when every slot
        // is small, else in s_perm
        const int* sorted = s_asg;
        if (!block_sort_small(s_asg, it.cnt, P, s_perm, s_cnt, s_off)) {
            block_sort_by_token(s_asg, it.cnt, P, s_perm, s_cnt, s_off);
            sorted = s_perm;
        }
        if (kDirect || it.kind == 1) {
            pool_slots_sorted(pa, b, off, P, sorted, s_off);
            return;
        }
        // gang: this shard's float64 partial sums per slot (members in
        // ascending order), published with a flag; then the G partials of
        // each slot are added in shard order
        double* __restrict__ part = a.gang_part + (size_t)(it.item0 + it.g) * P * C1;
        int32_t* __restrict__ cnts = a.shard_cells + (size_t)(it.item0 + it.g) * (P + 1);
        for (int j = tid; j < P; j += kFpsT) {
            const int beg = s_off[j], end = s_off[j + 1];
            cnts[j] = end - beg;
            double* __restrict__ pj = part + (size_t)j * C1;
            for (int c0 = 0; c0 < C; c0 += kPoolCols) {
                const int nc = min(kPoolCols, C - c0);
                double W, Sx[kPoolCols];
                pool_slot(pa, off, beg, end, c0, nc, [&](int m) { return it.lo + sorted[m]; }, W,
                          Sx);
                if (c0 == 0) pj[0] = W;
#pragma unroll
                for (int q = 0; q < kPoolCols; ++q)
                    if (q < nc) pj[1 + c0 + q] = Sx[q];
            }
        }
    }
    __threadfence();
    __syncthreads();
    // the flag is word 0 of this shard's record of the parity no exchange
    // reads any more, tag P+1 (exchange tags are at most P-1)
    unsigned long long* rec = a.gang_rec + (size_t)it.item0 * 2 * kGangRecWords;
    const int par = it.par;
    if (tid == 0)
        __hip_atomic_store(rec + ((size_t)it.g * 2 + par) * kGangRecWords, rec_word(P + 1, 0, 0),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    {
        const int lane = lane_id();
        const uint32_t want = (uint32_t)(P + 1);
        for (uint32_t spin = 0;; ++spin) {
            bool ok = true;
            for (int q = lane; q < it.G; q += 64) {
                const unsigned long long w = __hip_atomic_load(
                    rec + ((size_t)q * 2 + par) * kGangRecWords, __ATOMIC_RELAXED,
                    __HIP_MEMORY_SCOPE_AGENT);
                ok = ok && rec_ok(w, (int)want);
            }
            if (ballot(!ok) == 0) break;
            if (spin >= a.spin_limit) {
                if (lane == 0)
                    __hip_atomic_fetch_or(a.header + 3, kErrPoolWait, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    __threadfence();
    // this workgroup's slots j = g, g+G, ...; one thread per (slot, column)
    // and one per slot for the member count; shard partials read 8 at a time
    const double* __restrict__ part0 = a.gang_part + (size_t)it.item0 * P * C1;
    const int32_t* __restrict__ cnts0 = a.shard_cells + (size_t)it.item0 * (P + 1);
    const int G = it.G;
    const int nmine = (P - it.g + G - 1) / G;
    for (int t = tid; t < nmine * C1; t += kFpsT) {
        const int js = t / C1;
        const int c = t - js * C1;
        const int j = it.g + G * js;
        if (c < C) {
            double W = 0.0, Sc = 0.0;
            for (int sh0 = 0; sh0 < G; sh0 += kBatch) {
                double w8[kBatch], s8[kBatch];
#pragma unroll
                for (int q = 0; q < kBatch; ++q) {
                    if (sh0 + q < G) {
                        const double* pj = part0 + ((size_t)(sh0 + q) * P + j) * C1;
                        w8[q] = pj[0];
                        s8[q] = pj[1 + c];
                    }
                }
#pragma unroll
                for (int q = 0; q < kBatch; ++q) {
                    if (sh0 + q < G) {
                        W += w8[q];
                        Sc += s8[q];
                    }
                }
            }
            pa.pooled[(b * P + j) * (int64_t)C + c] = W != 0.0 ? (float)(Sc / W) : 0.0f;
        } else if (pa.cell_count) {
            int count = 0;
            for (int sh0 = 0; sh0 < G; sh0 += kBatch) {
                int c8[kBatch];
#pragma unroll
                for (int q = 0; q < kBatch; ++q)
                    c8[q] = sh0 + q < G ? cnts0[(size_t)(sh0 + q) * (P + 1) + j] : 0;
#pragma unroll
                for (int q = 0; q < kBatch; ++q) count += c8[q];
            }
            pa.cell_count[b * P + j] = count;
        }
    }
}

// ------------------------------------------------ token packing (next)

__device__ __forceinline__ int clamp_count(int t, int P) { return t < 0 ? 0 : (t > P ? P : t); }

// cu[b] = T_0 + ... + T_{b-1} (counts clamped into [0, P]), cu[B] = the
// total.  One workgroup of 1024 threads, 1024 events per round.
__global__ __launch_bounds__(1024) void pack_scan_kernel(const int32_t* __restrict__ tc, int64_t B,
                                                         int P, int32_t* __restrict__ cu) {
    __shared__ int s_w[16];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    int carry = 0;
    for (int64_t base = 0; base < B; base += 1024) {
        const int64_t b = base + tid;
        const int t = b < B ? clamp_count(tc[b], P) : 0;
        const int incl = wave_incl_scan(t);
        if (lane == 63) s_w[wave] = incl;
        __syncthreads();
        int wb = 0, total = 0;
        for (int w = 0; w < 16; ++w) {
            const int v = s_w[w];
            wb += w < wave ? v : 0;
            total += v;
        }
        if (b < B) cu[b] = carry + wb + incl - t;
        carry += total;
        __syncthreads();
    }
    if (tid == 0) cu[B] = carry;
}

// Event b's first T_b rows of D floats (one contiguous block) to packed rows
// cu[b] ..; block (bx, by): bx threads along a row, by rows at a time.
__global__ __launch_bounds__(256) void pack_copy_kernel(const int32_t* __restrict__ tc, int P, int D,
                                                        const int32_t* __restrict__ cu,
                                                        const float* __restrict__ rows,
                                                        float* __restrict__ packed,
                                                        int32_t* __restrict__ doc_id) {
    const int64_t b = blockIdx.x;
    const int T = clamp_count(tc[b], P);
    const int64_t at = cu[b];
    const float* __restrict__ src = rows + b * (int64_t)P * D;
    float* __restrict__ dst = packed + at * D;
    for (int j = threadIdx.y; j < T; j += blockDim.y)
        for (int d = threadIdx.x; d < D; d += blockDim.x)
            dst[(int64_t)j * D + d] = src[(int64_t)j * D + d];
    if (doc_id) {
        const int nt = blockDim.x * blockDim.y;
        for (int j = threadIdx.y * blockDim.x + threadIdx.x; j < T; j += nt)
            doc_id[at + j] = (int32_t)b;
    }
}

// rows[b][j] = packed[cu[b] + j] for j < T_b, else 0.
__global__ __launch_bounds__(256) void unpack_kernel(const int32_t* __restrict__ tc, int P, int D,
                                                     const int32_t* __restrict__ cu,
                                                     const float* __restrict__ packed,
                                                     float* __restrict__ rows) {
    const int64_t b = blockIdx.x;
    const int T = clamp_count(tc[b], P);
    const float* __restrict__ src = packed + (int64_t)cu[b] * D;
    float* __restrict__ dst = rows + b * (int64_t)P * D;
    for (int j = threadIdx.y; j < P; j += blockDim.y)
        for (int d = threadIdx.x; d < D; d += blockDim.x)
            dst[(int64_t)j * D + d] = j < T ? src[(int64_t)j * D + d] : 0.0f;
}

// ---------------------------------------------- pooling backward (next)

// One token's contribution to column c of member i's gradient: g[c] * w_i /
// W, then, for the weight column, (sum over c2 of g[c2] * (f_i[c2] - m[c2]))
// / W, in float64 with no contraction.  g, m: the token's rows (LDS or
// device memory), f: the member's feature row.
__device__ __forceinline__ double bwd_token(const float* __restrict__ g,
                                           const float* __restrict__ m,
                                           const float* __restrict__ f, int C, int wcol,
                                           double W, double wi, int c, double acc) {
    acc = acc + (double)g[c] * wi / W;
    if (c == wcol) {
        double s = 0.0;
        for (int c2 = 0; c2 < C; ++c2) s = s + (double)g[c2] * ((double)f[c2] - (double)m[c2]);
        acc = acc + s / W;
    }
    return acc;
}

// The same with the member's row in registers (C <= kPoolCols): identical
// float64 operations in the same order.
__device__ __forceinline__ double bwd_token_r(const float* __restrict__ g,
                                             const float* __restrict__ m,
                                             const float (&fr)[kPoolCols], int C, int wcol,
                                             double W, double wi, int c, double acc) {
    acc = acc + (double)g[c] * wi / W;
    if (c == wcol) {
        // the token's two rows loaded whole before the sum
        float gr[kPoolCols], mr[kPoolCols];
#pragma unroll
        for (int c2 = 0; c2 < kPoolCols; ++c2) {
            gr[c2] = g[min(c2, C - 1)];
            mr[c2] = m[min(c2, C - 1)];
        }
        double s = 0.0;
#pragma unroll
        for (int c2 = 0; c2 < kPoolCols; ++c2)
            if (c2 < C) s = s + (double)gr[c2] * ((double)fr[c2] - (double)mr[c2]);
        acc = acc + s / W;
    }
    return acc;
}

// A member's feature row in registers, every load issued together.
__device__ __forceinline__ void bwd_row(const float* __restrict__ f, int C, float (&fr)[kPoolCols]) {
#pragma unroll
    for (int c = 0; c < kPoolCols; ++c) fr[c] = f[min(c, C - 1)];
}

// The member's weight (1 without a weight column).  The load is issued
// either way (column 0 then), so a batch of them is not serialised behind
// the test.
__device__ __forceinline__ double bwd_weight(const PoolBwdArgs& a, int64_t row) {
    const float v = a.features[row * a.C + (a.wcol >= 0 ? a.wcol : 0)];
    return a.wcol >= 0 ? (double)v : 1.0;
}

// Voronoi: each pulse's one token.  G, M: the event's token rows [T][C].
__device__ __forceinline__ void bwd_pulses_voronoi(const PoolBwdArgs& a, int64_t off, int n,
                                                   int T, const double* s_W,
                                                   const float* __restrict__ G,
                                                   const float* __restrict__ M) {
    const int C = a.C;
    for (int64_t i = threadIdx.x; i < n; i += kSortT) {
        const int j = a.assign[off + i];
        const bool in = T >= 1 && j >= 0 && j < T && s_W[j] != 0.0;
        const double W = in ? s_W[j] : 1.0;
        const double wi = bwd_weight(a, off + i);
        const float* __restrict__ f = a.features + (off + i) * C;
        const int jj = in ? j : 0;
        float* __restrict__ out = a.grad + (off + i) * C;
        if (C <= kPoolCols) {
            float fr[kPoolCols];
            bwd_row(f, C, fr);
            for (int c = 0; c < C; ++c)
                out[c] = (float)(in ? bwd_token_r(G + (int64_t)jj * C, M + (int64_t)jj * C, fr, C,
                                                  a.wcol, W, wi, c, 0.0)
                                    : 0.0);
        } else {
            for (int c = 0; c < C; ++c)
                out[c] = (float)(in ? bwd_token(G + (int64_t)jj * C, M + (int64_t)jj * C, f, C,
                                                a.wcol, W, wi, c, 0.0)
                                    : 0.0);
        }
    }
}

// kNN: each pulse's tokens in ascending order, from its words of the token
// bitmap (bits: [n][PW] in LDS, or NULL: scan every list).
__device__ __forceinline__ void bwd_pulses_knn(const PoolBwdArgs& a, int64_t off, int n, int T,
                                               const double* s_W, const float* __restrict__ G,
                                               const float* __restrict__ M,
                                               const uint32_t* bits, int PW,
                                               const int32_t* __restrict__ lists) {
    const int C = a.C;
    const int k = a.k;
    for (int64_t i = threadIdx.x; i < n; i += kSortT) {
        const double wi = bwd_weight(a, off + i);
        const float* __restrict__ f = a.features + (off + i) * C;
        float* __restrict__ out = a.grad + (off + i) * C;
        uint32_t tw[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) tw[w] = bits && w < PW ? bits[i * PW + w] : 0u;
        if (bits && PW <= 4 && C <= kPoolCols) {
            // narrow rows: tokens outer, columns inner, one float64 sum per
            // column in registers (each column's additions keep ascending
            // token order); each token's rows are read once
            float fr[kPoolCols];
            bwd_row(f, C, fr);
            double acc[kPoolCols];
#pragma unroll
            for (int c = 0; c < kPoolCols; ++c) acc[c] = 0.0;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t bw = tw[w];
                while (bw) {
                    const int j = (w << 5) + (int)__builtin_ctz(bw);
                    bw &= bw - 1u;
                    const double W = s_W[j];
                    if (W == 0.0) continue;
                    const float* __restrict__ g = G + (int64_t)j * C;
                    const float* __restrict__ m = M + (int64_t)j * C;
                    float gr[kPoolCols], mr[kPoolCols];
#pragma unroll
                    for (int c = 0; c < kPoolCols; ++c) {
                        gr[c] = g[min(c, C - 1)];
                        mr[c] = m[min(c, C - 1)];
                    }
#pragma unroll
                    for (int c = 0; c < kPoolCols; ++c)
                        if (c < C) acc[c] = acc[c] + (double)gr[c] * wi / W;
                    if (a.wcol >= 0) {
                        double sw = 0.0;
#pragma unroll
                        for (int c = 0; c < kPoolCols; ++c)
                            if (c < C) sw = sw + (double)gr[c] * ((double)fr[c] - (double)mr[c]);
#pragma unroll
                        for (int c = 0; c < kPoolCols; ++c)
                            if (c == a.wcol) acc[c] = acc[c] + sw / W;
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < kPoolCols; ++c)
                if (c < C) out[c] = (float)acc[c];
            continue;
        }
        for (int c = 0; c < C; ++c) {
            double acc = 0.0;
            if (bits && PW <= 4) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    uint32_t bw = tw[w];
                    while (bw) {
                        const int j = (w << 5) + (int)__builtin_ctz(bw);
                        bw &= bw - 1u;
                        if (s_W[j] != 0.0)
                            acc = bwd_token(G + (int64_t)j * C, M + (int64_t)j * C, f, C, a.wcol,
                                            s_W[j], wi, c, acc);
                    }
                }
            } else if (bits) {
                for (int w = 0; w < PW; ++w) {
                    uint32_t bw = bits[i * PW + w];
                    while (bw) {
                        const int j = (w << 5) + (int)__builtin_ctz(bw);
                        bw &= bw - 1u;
                        if (s_W[j] != 0.0)
                            acc = bwd_token(G + (int64_t)j * C, M + (int64_t)j * C, f, C, a.wcol,
                                            s_W[j], wi, c, acc);
                    }
                }
            } else {
                for (int j = 0; j < T; ++j) {
                    bool hit = false;
                    for (int e = 0; e < k; ++e) hit = hit || lists[(int64_t)j * k + e] == (int)i;
                    if (hit && s_W[j] != 0.0)
                        acc = bwd_token(G + (int64_t)j * C, M + (int64_t)j * C, f, C, a.wcol,
                                        s_W[j], wi, c, acc);
                }
            }
            out[c] = (float)acc;
        }
    }
}

// Gradient of the pooling with respect to the features, one workgroup per
// event.  Token weight sums W_j first (float64, member order: Voronoi
// members sorted by slot, stable, so ascending; kNN lists in list order, k
// entries loaded together), then one thread per pulse adds, column by
// column, the contributions of the tokens that hold it, in ascending token
// order.  The event's grad_pooled and pooled rows are copied to LDS (the
// sort's permutation area, free by then) when they fit.  kNN mode finds a
// pulse's tokens in a per-pulse bitmap over the tokens (dynamic LDS,
// a.bits_cap words) when it fits, else by scanning every list.
__global__ __launch_bounds__(kSortT) void pool_backward_kernel(PoolBwdArgs a) {
    __shared__ double s_W[kMaxP];
    __shared__ int s_cnt[kSortW * kMaxP];
    __shared__ int s_off[kMaxP + 1];
    __shared__ __align__(16) int s_perm[kLdsPerm];
    extern __shared__ uint32_t s_bits[];
    const int64_t b = blockIdx.x;
    int64_t off;
    int n;
    event_range(a.offsets, a.N, b, off, n);
    if (n == 0) return;
    const int tid = threadIdx.x;
    const int P = a.P;
    const int C = a.C;
    const int T = clamp_count(a.token_count[b], P);
    const int k = a.k;
    const int32_t* __restrict__ lists = a.knn_idx ? a.knn_idx + b * (int64_t)P * k : nullptr;
    const int PW = (P + 31) >> 5;
    const bool use_bits = a.mode == 1 && (int64_t)n * PW <= a.bits_cap;
    if (a.mode == 0) {
        if (T >= 1) {
            int* perm = n <= kLdsPerm ? s_perm : a.perm + off;
            block_sort_by_token<true>(a.assign + off, n, T, perm, s_cnt, s_off);
            for (int j = tid; j < T; j += kSortT) {
                // kBatch weights loaded together, added in member order (a
                // padded batch adds +0.0, which leaves the sum unchanged)
                double W = 0.0;
                const int e = s_off[j + 1];
                for (int m0 = s_off[j]; m0 < e; m0 += kBatch) {
                    double wv[kBatch];
#pragma unroll
                    for (int q = 0; q < kBatch; ++q) {
                        // past the slot: member e-1 re-read, its weight unused
                        const double v = bwd_weight(a, off + perm[min(m0 + q, e - 1)]);
                        wv[q] = m0 + q < e ? v : 0.0;
                    }
#pragma unroll
                    for (int q = 0; q < kBatch; ++q) W = W + wv[q];
                }
                s_W[j] = W;
            }
        }
    } else {
        if (use_bits) {
            for (int64_t q = tid; q < (int64_t)n * PW; q += kSortT) s_bits[q] = 0u;
            __syncthreads();
        }
        for (int j = tid; j < T; j += kSortT) {
            double W = 0.0;
            for (int e0 = 0; e0 < k; e0 += kBatch) {
                int iv[kBatch];
#pragma unroll
                for (int q = 0; q < kBatch; ++q) iv[q] = e0 + q < k ? lists[(int64_t)j * k + e0 + q] : -1;
                double wv[kBatch];
#pragma unroll
                for (int q = 0; q < kBatch; ++q) {
                    // a missing entry reads row 0, its weight unused
                    const bool ok = iv[q] >= 0 && iv[q] < n;
                    const double v = bwd_weight(a, off + (ok ? iv[q] : 0));
                    wv[q] = ok ? v : 0.0;
                }
#pragma unroll
                for (int q = 0; q < kBatch; ++q) W = W + wv[q];
                if (use_bits) {
#pragma unroll
                    for (int q = 0; q < kBatch; ++q)
                        if (iv[q] >= 0 && iv[q] < n)
                            atomicOr(&s_bits[(int64_t)iv[q] * PW + (j >> 5)], 1u << (j & 31));
                }
            }
            s_W[j] = W;
        }
    }
    __syncthreads();
    // the event's token rows, in LDS when both fit the permutation area
    const float* G = a.grad_pooled + b * (int64_t)P * C;
    const float* M = a.pooled + b * (int64_t)P * C;
    const bool stage = 2 * (int64_t)T * C <= kLdsPerm;
    if (stage) {
        float* sg = reinterpret_cast<float*>(s_perm);
        for (int q = tid; q < T * C; q += kSortT) {
            sg[q] = G[q];
            sg[T * C + q] = M[q];
        }
    }
    __syncthreads();
    const uint32_t* bits = use_bits ? s_bits : nullptr;
    if (stage) {
        const float* sg = reinterpret_cast<const float*>(s_perm);
        if (a.mode == 0)
            bwd_pulses_voronoi(a, off, n, T, s_W, sg, sg + T * C);
        else
            bwd_pulses_knn(a, off, n, T, s_W, sg, sg + T * C, bits, PW, lists);
    } else {
        if (a.mode == 0)
            bwd_pulses_voronoi(a, off, n, T, s_W, G, M);
        else
            bwd_pulses_knn(a, off, n, T, s_W, G, M, bits, PW, lists);
    }
}

// -------------------------------------------- low-precision inputs (next)

// The float32 value of a 16-bit input element: binary16 through the
// hardware conversion (exact: every binary16 value is a float32 value),
// bfloat16 as the upper half of a float32.
__device__ __forceinline__ float upcast16(uint16_t h, int dtype) {
    return dtype == 1 ? (float)__builtin_bit_cast(_Float16, h) : __uint_as_float((uint32_t)h << 16);
}

// dst_a[i] = upcast16(src_a[i]) for i < na, then the same for b, one
// grid-stride pass over both arrays; four elements per thread and step (one
// 8-byte load when the array is 8-byte aligned, which 16-bit coordinates
// are), single elements at the ends.
__global__ __launch_bounds__(256) void upcast_kernel(const uint16_t* __restrict__ sa, int64_t na,
                                                     int da, float* __restrict__ oa,
                                                     const uint16_t* __restrict__ sb, int64_t nb,
                                                     int db, float* __restrict__ ob) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
    for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < na + nb;
         i += stride) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t q = i + u;
            if (q < na)
                oa[q] = upcast16(sa[q], da);
            else if (q < na + nb)
                ob[q - na] = upcast16(sb[q - na], db);
        }
    }
}

hipError_t launch_upcast(const void* src_a, int64_t na, int dtype_a, float* dst_a,
                         const void* src_b, int64_t nb, int dtype_b, float* dst_b, hipStream_t s) {
    const int64_t total = na + nb;
    if (total <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((total + 1023) / 1024, 8192);
    hipLaunchKernelGGL(upcast_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       (const uint16_t*)src_a, na, dtype_a, dst_a, (const uint16_t*)src_b, nb,
                       dtype_b, dst_b);
    return hipGetLastError();
}

// ----------------------------------------------- random FPS start (next)

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC 2011): ten rounds, each
// two 32x32 -> 64-bit products of counter words 0 and 2 with 0xD2511F53 and
// 0xCD9E8D57, their halves crossed with words 1 and 3 and the key; the key
// advances by 0x9E3779B9 and 0xBB67AE85 between rounds.  Returns word 0.
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c0;
}

// start_idx[b] = floor(u_b * n_b / 2^32), u_b = word 0 of the block at
// counter (b, step) and key seed; one thread per event.
__global__ __launch_bounds__(256) void random_start_kernel(const int64_t* __restrict__ offsets,
                                                           int64_t B, uint64_t seed, uint64_t step,
                                                           int32_t* __restrict__ start_idx) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= B) return;
    const int64_t n = offsets[b + 1] - offsets[b];
    const uint32_t u = philox_word0((uint32_t)b, (uint32_t)((uint64_t)b >> 32), (uint32_t)step,
                                    (uint32_t)(step >> 32), (uint32_t)seed, (uint32_t)(seed >> 32));
    start_idx[b] = n > 0 ? (int32_t)(((uint64_t)u * (uint64_t)n) >> 32) : 0;
}

// ------------------------------------------- no-allocation scratch region

// The workspace of fpstok_tokenize_noalloc, for callers that cannot allocate
// device memory: one fixed region per GPU, a file-scope device array that
// every GPU the library runs on holds until the process ends.  Host code never
// uses the array's name as an address (on the host it is only a stand-in for
// the symbol): noalloc_scratch looks the device address up with
// hipGetSymbolAddress once per device, with that device current, and every
// launch takes that address.
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;

hipError_t noalloc_scratch(void** ptr) {
    static std::mutex mu;
    static void* by_device[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!by_device[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || ((uintptr_t)p & 255u) != 0) return hipErrorInvalidSymbol;
        by_device[dev] = p;
    }
    *ptr = by_device[dev];
    return hipSuccess;
}

// ------------------------------------------------------------------ launchers

static inline unsigned grid1(int64_t x) { return (unsigned)(x < 1 ? 1 : x); }

// Compute units of the current device (cached per device; 256 if unknown).
static int device_cus() {
    static std::mutex mu;
    static int by_device[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (by_device[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n < 1)
            n = 256;
        by_device[dev] = n;
    }
    return by_device[dev];
}

hipError_t launch_plan(const int64_t* offsets, int64_t B, int64_t N, void* ws,
                       const WorkspaceLayout& L, hipStream_t s) {
    char* base = (char*)ws;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, offsets, B, N, L.max_chunks,
                       (int32_t*)(base + L.header), (int32_t*)(base + L.chunk_ev),
                       (int32_t*)(base + L.chunk_beg));
    return hipGetLastError();
}

// Chunk-list length above which the planner orders the partial chunks by
// length: the persistent sorting kernel takes the list in rounds of one chunk
// per compute unit; the other pooling kernel takes one chunk per workgroup.
static int64_t pool_band_over(const PoolArgs& a) {
    return a.P <= kSrtMaxP && a.C <= kSrtMaxC ? (int64_t)device_cus() : INT64_MAX;
}

// Whether a batch's chunk list can be longer than band_over: every event
// makes at most n / kPoolChunk + 1 chunks.
static bool pool_bands(int64_t B, int64_t N, int64_t band_over) {
    return B + N / kPoolChunk > band_over;
}

hipError_t launch_plan_pool(const int64_t* offsets, int64_t B, int64_t N, void* ws,
                            const WorkspaceLayout& L, const PoolArgs& a, hipStream_t s) {
    char* base = (char*)ws;
    const int64_t over = pool_band_over(a);
    auto k = pool_bands(B, N, over) ? plan_pool_kernel<true> : plan_pool_kernel<false>;
    hipLaunchKernelGGL(k, dim3(1), dim3(1024), 0, s, offsets, B, N, L.max_pool_chunks,
                       L.max_parts, (int32_t*)(base + L.header), (int32_t*)(base + L.pool_ev),
                       (int32_t*)(base + L.pool_beg), (int32_t*)(base + L.chunk_part),
                       (int32_t*)(base + L.big_ev), a.whole, over);
    return hipGetLastError();
}

hipError_t launch_pool_combine(const PoolArgs& a, hipStream_t s) {
    if (a.whole) return hipSuccess;
    // events of more than one chunk hold more than kPoolChunk pulses
    const int64_t big = std::min<int64_t>(a.B, a.N / ((int64_t)kPoolChunk + 1));
    if (big <= 0) return hipSuccess;
    const int C2 = a.C + 2;
    const int spg = 256 / C2;
    hipLaunchKernelGGL(pool_combine_kernel, dim3((unsigned)big, (unsigned)((a.P + spg - 1) / spg)),
                       dim3(C2, spg), 0, s, a);
    return hipGetLastError();
}

int64_t sample_max_items(int64_t B, int64_t N) { return B + N / kFpsCap; }

hipError_t launch_plan_all(const SampleArgs& a, int64_t B, void* ws, const WorkspaceLayout& L,
                           const PoolArgs& pa, bool chunks, bool pool, hipStream_t s) {
    char* base = (char*)ws;
    const int64_t over = pool_band_over(pa);
    auto k = pool && pool_bands(B, a.N, over) ? plan_all_kernel<true> : plan_all_kernel<false>;
    hipLaunchKernelGGL(k, dim3(1), dim3(1024), 0, s, a, B, (int32_t*)(base + L.chunk_ev),
                       (int32_t*)(base + L.chunk_beg), L.max_chunks, pa, L.max_pool_chunks,
                       L.max_parts, chunks ? 1 : 0, pool ? 1 : 0, over);
    return hipGetLastError();
}

hipError_t launch_sample_items(const SampleArgs& a, int64_t B, hipStream_t s) {
    hipLaunchKernelGGL(sample_kernel, dim3(grid1(sample_max_items(B, a.N))), dim3(kFpsT), 0, s, a);
    return hipGetLastError();
}

// Threads of the FPS work-list kernel: one per event, whole waves, up to 1024.
static unsigned plan_fps_threads(int64_t B) {
    return (unsigned)(B >= 1024 ? 1024 : ((B + 63) / 64) * 64);
}

hipError_t launch_sample(const SampleArgs& a, int64_t B, hipStream_t s) {
    if (!a.direct) {
        hipLaunchKernelGGL(plan_fps_kernel, dim3(1), dim3(plan_fps_threads(B)), 0, s, a, B);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sample_kernel, dim3(grid1(a.direct ? B : sample_max_items(B, a.N))),
                       dim3(kFpsT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_tokenize(const SampleArgs& a, const PoolArgs& pa, int64_t B, hipStream_t s) {
    if (!a.direct) {
        hipLaunchKernelGGL(plan_fps_kernel, dim3(1), dim3(plan_fps_threads(B)), 0, s, a, B);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // feature rows of small single-workgroup events are staged in LDS when
    // that leaves two workgroups per CU their room
    PoolArgs p = pa;
    p.stage_cap = a.P <= 512 ? kStage : 0;
    const size_t lds = sizeof(int) * ((size_t)kSortW * a.P + a.P + 1 + 2 * (size_t)kFpsCap) +
                       sizeof(float) * (size_t)p.stage_cap;
    if (a.direct)
        hipLaunchKernelGGL(tokenize_kernel<true>, dim3(grid1(B)), dim3(kFpsT), lds, s, a, p);
    else
        hipLaunchKernelGGL(tokenize_kernel<false>, dim3(grid1(sample_max_items(B, a.N))),
                           dim3(kFpsT), lds, s, a, p);
    return hipGetLastError();
}

hipError_t launch_assign(const AssignArgs& a, int64_t max_chunks, hipStream_t s) {
    hipLaunchKernelGGL(assign_kernel, dim3(grid1(max_chunks)), dim3(kAsgT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_knn(const KnnArgs& a, int64_t B, hipStream_t s) {
    const int64_t nb = (a.P + kKnnW - 1) / kKnnW;
    hipLaunchKernelGGL(knn_kernel, dim3(grid1(B * nb)), dim3(kKnnT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_lloyd_update(const LloydArgs& a, int64_t B, hipStream_t s) {
    const size_t lds = (sizeof(float4) + sizeof(float) + sizeof(int)) * (size_t)(kLdsPerm + 1);
    hipLaunchKernelGGL(lloyd_update_kernel, dim3(grid1(B)), dim3(kSortT), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_pool_voronoi(const PoolArgs& a, int64_t max_chunks, hipStream_t s) {
    if (a.P <= kSrtMaxP && a.C <= kSrtMaxC) {
        // rows sorted by slot into LDS; one persistent workgroup per compute unit
        const size_t lds = sizeof(float) * ((size_t)kPoolChunk * a.C + kSrtZero) +
                           sizeof(int) * ((size_t)kSrtW * a.P + ((a.P + 2) & ~1)) +
                           sizeof(unsigned long long) * (size_t)kSrtW * a.P;
        const dim3 g((unsigned)std::max<int64_t>(1, std::min<int64_t>(max_chunks, device_cus()))),
            t(kSrtT);
        switch (a.C) {
            case 1: hipLaunchKernelGGL(pool_sorted_kernel<1>, g, t, lds, s, a); break;
            case 2: hipLaunchKernelGGL(pool_sorted_kernel<2>, g, t, lds, s, a); break;
            case 3: hipLaunchKernelGGL(pool_sorted_kernel<3>, g, t, lds, s, a); break;
            case 4: hipLaunchKernelGGL(pool_sorted_kernel<4>, g, t, lds, s, a); break;
            case 5: hipLaunchKernelGGL(pool_sorted_kernel<5>, g, t, lds, s, a); break;
            default: hipLaunchKernelGGL(pool_sorted_kernel<6>, g, t, lds, s, a); break;
        }
        return hipGetLastError();
    }
    const size_t lds = sizeof(unsigned long long) * kSortW * (size_t)a.P +
                       sizeof(int) * (2 * (size_t)kPoolChunk + kSortW * (size_t)a.P + a.P + 1);
    hipLaunchKernelGGL(pool_chunk_kernel, dim3(grid1(max_chunks)), dim3(kSortT), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_pool_knn(const PoolArgs& a, int64_t B, hipStream_t s) {
    hipLaunchKernelGGL(pool_knn_kernel, dim3(grid1(B)), dim3(kSortT), 0, s, a);
    return hipGetLastError();
}

static dim3 row_block(int D) {
    const int bx = D < 256 ? D : 256;
    return dim3((unsigned)bx, (unsigned)(256 / bx));
}

hipError_t launch_pack(int64_t B, int P, int D, const int32_t* tc, const float* rows,
                       float* packed, int32_t* doc_id, int32_t* cu, hipStream_t s) {
    hipLaunchKernelGGL(pack_scan_kernel, dim3(1), dim3(1024), 0, s, tc, B, P, cu);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || B == 0) return e;
    hipLaunchKernelGGL(pack_copy_kernel, dim3((unsigned)B), row_block(D), 0, s, tc, P, D,
                       (const int32_t*)cu, rows, packed, doc_id);
    return hipGetLastError();
}

hipError_t launch_unpack(int64_t B, int P, int D, const int32_t* tc, const int32_t* cu,
                         const float* packed, float* rows, hipStream_t s) {
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)B), row_block(D), 0, s, tc, P, D, cu, packed,
                       rows);
    return hipGetLastError();
}

hipError_t launch_random_start(const int64_t* offsets, int64_t B, uint64_t seed, uint64_t step,
                               int32_t* start_idx, hipStream_t s) {
    hipLaunchKernelGGL(random_start_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s,
                       offsets, B, seed, step, start_idx);
    return hipGetLastError();
}

hipError_t launch_pool_backward(const PoolBwdArgs& a, int64_t B, hipStream_t s) {
    PoolBwdArgs p = a;
    p.bits_cap = a.mode == 1 ? kBwdBitsCap : 0;
    const size_t lds = sizeof(uint32_t) * (size_t)p.bits_cap;
    hipLaunchKernelGGL(pool_backward_kernel, dim3(grid1(B)), dim3(kSortT), lds, s, p);
    return hipGetLastError();
}

}  // namespace fpstok
