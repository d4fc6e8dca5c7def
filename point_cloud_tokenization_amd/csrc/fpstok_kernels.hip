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

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(dpp_i<CTRL, ROW_MASK>(__float_as_int(v)));
}

// DPP controls (gfx9 family): quad permutes, row mirrors, row broadcasts.
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowMirror = 0x140;
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;

__device__ __forceinline__ int wave_min_i(int v) {
    v = min(v, dpp_i<kQuadSwap1, 0xF>(v));
    v = min(v, dpp_i<kQuadSwap2, 0xF>(v));
    v = min(v, dpp_i<kRowHalfMirror, 0xF>(v));
    v = min(v, dpp_i<kRowMirror, 0xF>(v));
    v = min(v, dpp_i<kRowBcast15, 0xA>(v));
    v = min(v, dpp_i<kRowBcast31, 0xC>(v));
    return readlane_i(v, 63);
}

__device__ __forceinline__ int wave_sum_i(int v) {
    v = v + dpp_i<kQuadSwap1, 0xF>(v);
    v = v + dpp_i<kQuadSwap2, 0xF>(v);
    v = v + dpp_i<kRowHalfMirror, 0xF>(v);
    v = v + dpp_i<kRowMirror, 0xF>(v);
    // rows hold their sums; combine the four row sums through readlane
    return readlane_i(v, 0) + readlane_i(v, 16) + readlane_i(v, 32) + readlane_i(v, 48);
}

// Inclusive prefix sum over the wave (Hillis-Steele with cross-lane shuffles).
__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
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
__global__ __launch_bounds__(1024) void plan_kernel(const int64_t* __restrict__ offsets,
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

// ---------------------------------------------------------------------- FPS

constexpr int kFpsT = 256;                 // threads per workgroup (4 waves)
constexpr int kFpsW = kFpsT / 64;
constexpr int kFpsM = 16;                  // register-resident pulses per thread
constexpr int kFpsCap = kFpsT * kFpsM;     // largest event kept in registers

struct __align__(16) FpsSlot {
    float v;
    int i;
    float pad0, pad1;
    float4 c;
};

// Workgroup-level argmax over the per-wave candidates written to `slots`:
// the largest value, then the lowest wave (waves hold increasing index
// ranges, so this is the lowest pulse index).  Values are compared as the
// int32 bit patterns of floats in {-1} U [0, inf], whose order they keep.
// Returns the winning slot uniformly.
__device__ __forceinline__ FpsSlot reduce_slots_blocked(const FpsSlot* slots) {
    const int lane = lane_id();
    const bool has = lane < kFpsW;
    FpsSlot s;
    if (has) s = slots[lane];
    const int v = has ? __float_as_int(s.v) : INT32_MIN;
    int r = max(v, dpp_i<kQuadSwap1, 0xF>(v));
    r = max(r, dpp_i<kQuadSwap2, 0xF>(r));
    const int gm = readlane_i(r, 0);
    const int L = (int)__builtin_ctzll(ballot(has && v == gm));
    FpsSlot out;
    out.v = __int_as_float(gm);
    out.i = readlane_i(s.i, L);
    out.c.x = readlane_f(s.c.x, L);
    out.c.y = readlane_f(s.c.y, L);
    out.c.z = readlane_f(s.c.z, L);
    out.c.w = readlane_f(s.c.w, L);
    return out;
}

__device__ __forceinline__ int wave_max_i(int v) {
    v = max(v, dpp_i<kQuadSwap1, 0xF>(v));
    v = max(v, dpp_i<kQuadSwap2, 0xF>(v));
    v = max(v, dpp_i<kRowHalfMirror, 0xF>(v));
    v = max(v, dpp_i<kRowMirror, 0xF>(v));
    v = max(v, dpp_i<kRowBcast15, 0xA>(v));
    v = max(v, dpp_i<kRowBcast31, 0xC>(v));
    return readlane_i(v, 63);
}

// FPS of one event with n in (P, 256*M], every pulse held in registers.
// Wave w owns the 64*M pulses starting at w*64*M; its register k of lane l
// holds pulse w*64*M + 64*k + l, so the loads are coalesced and the lowest
// pulse index among ties is the lowest lane of the lowest register (then the
// lowest wave) holding the maximum.
//
// Per pulse and iteration: the float32 distance to the newest centroid (11
// VALU ops), the fused Voronoi update (compare + 2 selects) and a share of a
// 3-input max.  Minimum distances are float32 values in {-1} U [0, inf]
// (-1 marks padding), compared as int32 bit patterns.
//
// Selected pulses are not marked: a selected pulse has min distance exactly
// 0, so while the maximum is > 0 it cannot win; when the maximum is 0 every
// pulse has min distance 0 and the rule "lowest unselected index" is applied
// from a selection bitmap over indices 0..2047 (the answer is < P <= 1024).
template <int M>
__device__ void fps_registers(const SampleArgs& a, int64_t b, int64_t off, int n, int s0) {
    __shared__ FpsSlot slots[2][kFpsW];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int P = a.P;
    const float4* __restrict__ p = a.coords + off;
    const int wbase = wave * 64 * M;

    float px[M], py[M], pz[M], pt[M], md[M];
    int nr[M];
#pragma unroll
    for (int k = 0; k < M; ++k) {
        const int i = wbase + 64 * k + lane;
        float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < n) q = p[i];
        px[k] = q.x;
        py[k] = q.y;
        pz[k] = q.z;
        pt[k] = q.w;
        md[k] = i < n ? INFINITY : -1.0f;  // padding never wins and is never updated
        nr[k] = 0;
    }

    uint32_t selbits = 0;
    int s = s0;
    float4 c = p[s];
    for (int j = 0; j < P; ++j) {
        if (tid == 0) {
            a.centroid_idx[b * P + j] = s;
            a.centroids[b * P + j] = c;
        }
        mark_selected(selbits, s);
        int bv = INT32_MIN;
#pragma unroll
        for (int k = 0; k < M; ++k) {
            const float d = sqd(px[k], py[k], pz[k], pt[k], c.x, c.y, c.z, c.w);
            const bool u = d < md[k];
            nr[k] = u ? j : nr[k];
            md[k] = u ? d : md[k];
            bv = max(bv, __float_as_int(md[k]));
        }
        if (j + 1 == P) break;

        const int wm = wave_max_i(bv);
        // lowest (register, lane) holding the wave maximum; every register
        // index is a compile-time constant, so no register indexing
        int wi = 0;
        float4 wc = make_float4(0.f, 0.f, 0.f, 0.f);
        bool found = false;
#pragma unroll
        for (int k = 0; k < M; ++k) {
            if (!found) {
                const uint64_t mk = ballot(__float_as_int(md[k]) == wm);
                if (mk != 0) {
                    found = true;
                    const int L = (int)__builtin_ctzll(mk);
                    wi = wbase + 64 * k + L;
                    wc = make_float4(readlane_f(px[k], L), readlane_f(py[k], L),
                                     readlane_f(pz[k], L), readlane_f(pt[k], L));
                }
            }
        }
        if (lane == 0) {
            FpsSlot& o = slots[j & 1][wave];
            o.v = __int_as_float(wm);
            o.i = wi;
            o.c = wc;
        }
        __syncthreads();
        const FpsSlot g = reduce_slots_blocked(slots[j & 1]);
        if (g.v == 0.0f) {
            s = min(first_unselected(selbits), n - 1);
            c = p[s];
        } else {
            s = min(max(g.i, 0), n - 1);
            c = g.c;
        }
    }
    if (a.assign) {
#pragma unroll
        for (int k = 0; k < M; ++k) {
            const int i = wbase + 64 * k + lane;
            if (i < n) a.assign[off + i] = nr[k];
        }
    }
}

// Register-resident FPS for m = ceil(n / 256) pulses per thread.
__device__ void fps_registers_dispatch(const SampleArgs& a, int64_t b, int64_t off, int n,
                                       int s0) {
    switch ((n + kFpsT - 1) / kFpsT) {
        case 1: fps_registers<1>(a, b, off, n, s0); break;
        case 2: fps_registers<2>(a, b, off, n, s0); break;
        case 3: fps_registers<3>(a, b, off, n, s0); break;
        case 4: fps_registers<4>(a, b, off, n, s0); break;
        case 5: fps_registers<5>(a, b, off, n, s0); break;
        case 6: fps_registers<6>(a, b, off, n, s0); break;
        case 7: fps_registers<7>(a, b, off, n, s0); break;
        case 8: fps_registers<8>(a, b, off, n, s0); break;
        case 9: case 10: fps_registers<10>(a, b, off, n, s0); break;
        case 11: case 12: fps_registers<12>(a, b, off, n, s0); break;
        case 13: case 14: fps_registers<14>(a, b, off, n, s0); break;
        default: fps_registers<16>(a, b, off, n, s0); break;
    }
}

// FPS of one event of any size, state streamed from the workspace (min
// distance) and from `assign` or the workspace (nearest slot) every
// iteration.  Thread t owns pulses t, t+256, ...; the argmax resolves ties
// by an explicit minimum over the index.
__device__ void fps_streaming(const SampleArgs& a, int64_t b, int64_t off, int n, int s0) {
    __shared__ FpsSlot slots[2][kFpsW];
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
        if (tid == 0) {
            a.centroid_idx[b * P + j] = s;
            a.centroids[b * P + j] = c;
        }
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
        int r = max(v, dpp_i<kQuadSwap1, 0xF>(v));
        r = max(r, dpp_i<kQuadSwap2, 0xF>(r));
        const float gm = __int_as_float(readlane_i(r, 0));
        const int gi = wave_min_i(has && v == __float_as_int(gm) ? sl.i : 0x7fffffff);
        s = gm == 0.0f ? first_unselected(selbits) : gi;
        s = min(max(s, 0), n - 1);
        c = p[s];
    }
}

__global__ __launch_bounds__(kFpsT) void sample_kernel(SampleArgs a) {
    const int64_t b = blockIdx.x;
    int64_t off;
    int n;
    event_range(a.offsets, a.N, b, off, n);
    const int P = a.P;
    const int tid = threadIdx.x;
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
        return;
    }
    int s0 = a.start_idx ? a.start_idx[b] : 0;
    if (s0 < 0 || s0 >= n) s0 = 0;
    if (n <= kFpsCap)
        fps_registers_dispatch(a, b, off, n, s0);
    else
        fps_streaming(a, b, off, n, s0);
    if (tid == 0) a.token_count[b] = P;
}

// ------------------------------------------------------------------- assign

constexpr int kAsgT = 256;
constexpr int kAsgR = kChunk / kAsgT;  // pulses per thread

// Nearest centroid of every pulse of one chunk; centroids staged in LDS and
// read as broadcasts; each thread keeps kAsgR pulses in registers.
__global__ __launch_bounds__(kAsgT) void assign_kernel(AssignArgs a) {
    __shared__ float4 s_c[1024];
    const int w = blockIdx.x;
    if (w >= a.header[0]) return;
    const int64_t b = a.chunk_ev[w];
    const int beg = a.chunk_beg[w];
    int64_t off;
    int n;
    event_range(a.offsets, a.N, b, off, n);
    if (n == 0 || (a.skip_small && n <= a.P)) return;
    int T = a.token_count[b];
    T = T > a.P ? a.P : T;
    if (T < 1) return;
    const int tid = threadIdx.x;
    for (int j = tid; j < T; j += kAsgT) s_c[j] = a.centroids[b * a.P + j];
    __syncthreads();
    const int end = min(n, beg + kChunk);
    float qx[kAsgR], qy[kAsgR], qz[kAsgR], qt[kAsgR], bd[kAsgR];
    int bj[kAsgR];
#pragma unroll
    for (int r = 0; r < kAsgR; ++r) {
        const int i = beg + tid + r * kAsgT;
        float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < end) q = a.coords[off + i];
        qx[r] = q.x;
        qy[r] = q.y;
        qz[r] = q.z;
        qt[r] = q.w;
        bd[r] = INFINITY;
        bj[r] = 0;
    }
    {
        const float4 c = s_c[0];
#pragma unroll
        for (int r = 0; r < kAsgR; ++r) bd[r] = sqd(qx[r], qy[r], qz[r], qt[r], c.x, c.y, c.z, c.w);
    }
    for (int j = 1; j < T; ++j) {
        const float4 c = s_c[j];
#pragma unroll
        for (int r = 0; r < kAsgR; ++r) {
            const float d = sqd(qx[r], qy[r], qz[r], qt[r], c.x, c.y, c.z, c.w);
            const bool u = d < bd[r];
            bd[r] = u ? d : bd[r];
            bj[r] = u ? j : bj[r];
        }
    }
#pragma unroll
    for (int r = 0; r < kAsgR; ++r) {
        const int i = beg + tid + r * kAsgT;
        if (i < end) a.assign[off + i] = bj[r];
    }
}

// ---------------------------------------------------------------------- kNN

constexpr int kKnnT = 256;
constexpr int kKnnW = kKnnT / 64;
constexpr int kKnnCap = 512;  // candidates per wave held in LDS

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
__global__ __launch_bounds__(kKnnT) void knn_kernel(KnnArgs a) {
    __shared__ uint64_t s_buf[kKnnW][kKnnCap];
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
    if (j >= T || n <= P) {
        for (int e = lane; e < k; e += 64) row[e] = (e == 0 && j < T && j < n) ? j : -1;
        return;
    }
    const float4 c = a.centroids[b * P + j];
    const float4* __restrict__ p = a.coords + off;

    uint64_t mykey = ~0ull;
    for (int i = lane; i < n; i += 64) {
        const float4 q = p[i];
        const uint64_t key = dkey(sqd(q.x, q.y, q.z, q.w, c.x, c.y, c.z, c.w), i);
        mykey = key < mykey ? key : mykey;
    }
    const int valid = min(n, 64);
    uint64_t tau = ~0ull;
    if (k <= valid) {
        int rank = 0;
        for (int l = 0; l < 64; ++l) {
            const uint64_t kl = ((uint64_t)(uint32_t)readlane_i((int)(mykey >> 32), l) << 32) |
                                (uint32_t)readlane_i((int)(uint32_t)mykey, l);
            rank += kl < mykey ? 1 : 0;
        }
        const int L = (int)__builtin_ctzll(ballot(rank == k - 1 && mykey != ~0ull));
        tau = ((uint64_t)(uint32_t)readlane_i((int)(mykey >> 32), L) << 32) |
              (uint32_t)readlane_i((int)(uint32_t)mykey, L);
    }
    uint64_t* __restrict__ buf = s_buf[wave];
    int cnt = 0;
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
    const int need = min(k, n);
    if (cnt <= kKnnCap) {
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        for (int q = lane; q < cnt; q += 64) {
            const uint64_t kq = buf[q];
            int rank = 0;
            for (int r = 0; r < cnt; ++r) rank += buf[r] < kq ? 1 : 0;
            if (rank < k) row[rank] = (int)(uint32_t)kq;
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
            if (lane == 0) row[e] = (int)(uint32_t)last;
        }
    }
    for (int e = need + lane; e < k; e += 64) row[e] = -1;
}

// ---------------------------------------------------- stable sort by token

constexpr int kSortT = 256;
constexpr int kSortW = kSortT / 64;
constexpr int kMaxP = 1024;

// Workgroup-wide stable counting sort of one event's pulses by slot:
// perm[s_off[j] + r] = the r-th pulse (ascending) with asg = j.  Pulses whose
// slot is outside [0, T) are left out.  Wave w handles the contiguous segment
// [w*seg, (w+1)*seg); inside a 64-pulse tile the rank of a pulse among equal
// slots comes from a bitwise ballot match, so the order is stable without
// atomics.  Two passes: count per (wave, slot), then place.
//   s_cnt: LDS int[kSortW * kMaxP];  s_off: LDS int[kMaxP + 1]
__device__ void block_sort_by_token(const int32_t* __restrict__ asg, int n, int T,
                                    int32_t* __restrict__ perm, int* s_cnt, int* s_off) {
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
            // block exclusive scan of `local`
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

// ------------------------------------------------------------ Lloyd update

// One workgroup per event with n > P: stable sort by slot, then every slot's
// charge-weighted mean in float64 over its members in ascending pulse order,
// rounded to float32; a zero-weight slot keeps its centroid.
__global__ __launch_bounds__(kSortT) void lloyd_update_kernel(LloydArgs a) {
    __shared__ int s_cnt[kSortW * kMaxP];
    __shared__ int s_off[kMaxP + 1];
    const int64_t b = blockIdx.x;
    int64_t off;
    int n;
    event_range(a.offsets, a.N, b, off, n);
    if (n <= a.P) return;
    int T = a.token_count[b];
    T = T > a.P ? a.P : T;
    if (T < 1) return;
    block_sort_by_token(a.assign + off, n, T, a.perm + off, s_cnt, s_off);
    const int32_t* __restrict__ perm = a.perm + off;
    for (int j = threadIdx.x; j < T; j += kSortT) {
        double W = 0.0, sx = 0.0, sy = 0.0, sz = 0.0, st = 0.0;
        const int e = s_off[j + 1];
        for (int q = s_off[j]; q < e; ++q) {
            const int i = perm[q];
            const double w = a.charge_col >= 0
                                 ? (double)a.features[(off + i) * (int64_t)a.C + a.charge_col]
                                 : 1.0;
            const float4 x = a.coords[off + i];
            W += w;
            sx += w * (double)x.x;
            sy += w * (double)x.y;
            sz += w * (double)x.z;
            st += w * (double)x.w;
        }
        if (W > 0.0)
            a.centroids[b * a.P + j] =
                make_float4((float)(sx / W), (float)(sy / W), (float)(sz / W), (float)(st / W));
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

// Voronoi pooling, one workgroup per event: stable sort by slot, then for
// every slot the (weighted) mean of its members in ascending pulse order.
__global__ __launch_bounds__(kSortT) void pool_voronoi_kernel(PoolArgs a) {
    __shared__ int s_cnt[kSortW * kMaxP];
    __shared__ int s_off[kMaxP + 1];
    const int64_t b = blockIdx.x;
    int64_t off;
    int n;
    event_range(a.offsets, a.N, b, off, n);
    int T = a.token_count[b];
    T = T < 0 ? 0 : (T > a.P ? a.P : T);
    if (T > 0) block_sort_by_token(a.assign + off, n, T, a.perm + off, s_cnt, s_off);
    const int32_t* __restrict__ perm = a.perm + off;
    const int C = a.C;
    for (int j = threadIdx.x; j < a.P; j += kSortT) {
        const int beg = j < T ? s_off[j] : 0;
        const int end = j < T ? s_off[j + 1] : 0;
        for (int c0 = 0; c0 < C; c0 += kPoolCols) {
            const int nc = min(kPoolCols, C - c0);
            double W = 0.0;
            double S[kPoolCols];
#pragma unroll
            for (int q = 0; q < kPoolCols; ++q) S[q] = 0.0;
            for (int m = beg; m < end; ++m) {
                const float* __restrict__ f = a.features + (off + perm[m]) * (int64_t)C;
                const double w = a.weight_col >= 0 ? (double)f[a.weight_col] : 1.0;
                W += w;
#pragma unroll
                for (int q = 0; q < kPoolCols; ++q)
                    if (q < nc) S[q] += w * (double)f[c0 + q];
            }
            pool_write(a, b, j, c0, nc, W, S);
        }
        if (a.cell_count) a.cell_count[b * a.P + j] = end - beg;
    }
}

// kNN pooling, one workgroup per event: every slot's list entries != -1 in
// list order.
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
        int count = 0;
        for (int c0 = 0; c0 < C; c0 += kPoolCols) {
            const int nc = min(kPoolCols, C - c0);
            double W = 0.0;
            double S[kPoolCols];
#pragma unroll
            for (int q = 0; q < kPoolCols; ++q) S[q] = 0.0;
            count = 0;
            if (j < T) {
                for (int e = 0; e < k; ++e) {
                    const int i = lst[e];
                    if (i < 0 || i >= n) continue;
                    const float* __restrict__ f = a.features + (off + i) * (int64_t)C;
                    const double w = a.weight_col >= 0 ? (double)f[a.weight_col] : 1.0;
                    W += w;
                    ++count;
#pragma unroll
                    for (int q = 0; q < kPoolCols; ++q)
                        if (q < nc) S[q] += w * (double)f[c0 + q];
                }
            }
            pool_write(a, b, j, c0, nc, W, S);
        }
        if (a.cell_count) a.cell_count[b * a.P + j] = count;
    }
}

// ------------------------------------------------------------------ launchers

static inline unsigned grid1(int64_t x) { return (unsigned)(x < 1 ? 1 : x); }

hipError_t launch_plan(const int64_t* offsets, int64_t B, int64_t N, void* ws,
                       const WorkspaceLayout& L, hipStream_t s) {
    char* base = (char*)ws;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, offsets, B, N, L.max_chunks,
                       (int32_t*)(base + L.header), (int32_t*)(base + L.chunk_ev),
                       (int32_t*)(base + L.chunk_beg));
    return hipGetLastError();
}

hipError_t launch_sample(const SampleArgs& a, int64_t B, hipStream_t s) {
    hipLaunchKernelGGL(sample_kernel, dim3(grid1(B)), dim3(kFpsT), 0, s, a);
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
    hipLaunchKernelGGL(lloyd_update_kernel, dim3(grid1(B)), dim3(kSortT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pool_voronoi(const PoolArgs& a, int64_t B, hipStream_t s) {
    hipLaunchKernelGGL(pool_voronoi_kernel, dim3(grid1(B)), dim3(kSortT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pool_knn(const PoolArgs& a, int64_t B, hipStream_t s) {
    hipLaunchKernelGGL(pool_knn_kernel, dim3(grid1(B)), dim3(kSortT), 0, s, a);
    return hipGetLastError();
}

}  // namespace fpstok
