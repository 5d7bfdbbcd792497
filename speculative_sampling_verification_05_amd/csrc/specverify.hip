// specverify.hip - batched speculative-sampling verification for gfx950.
//
// Pages (cited by title and section):
//  [Ch15] "Chapter 15: Decoding acceleration techniques" (zsc.github.io, LLM
//         edge inference), 15.1.2: step 2 (softmax of every verified row),
//         step 3 (accept with probability min(1, p/q), stop at the first
//         rejection), step 4 (resample from max(0, p - q)/Z); 15.1.4 (the
//         probability gather); 15.4.2 (fused kernels, low-precision inputs
//         with fp32 accumulation, coalesced loads).
//  [CSDN] devpress.csdn.net speculative-inference post, 2.1: the
//         speculative_decode() loop (strict u < alpha, residual clamp).
//  [HSD]  "LLM inference optimisation: hidden-state speculative decoding", 3.3:
//         the bonus token drawn from the last target row.
//
// One kernel launch per call. Its grid holds two kinds of 256-thread blocks,
// laid out group by group (a group is one sequence; for the stand-alone row
// statistics it is one row):
//  statistics blocks  stream the group's rows once (all the compulsory bytes).
//                     Each wavefront owns a contiguous range of 1 KiB chunks of
//                     the group's concatenated rows, keeps per lane an online
//                     max and a sum of 2^(x*c - R) (R an integer reference,
//                     c = log2(e)/T), software-pipelines its 16-byte loads and
//                     writes one partial per row piece; at T == 0 it tracks the
//                     argmax (first index of the maximum) instead. Each
//                     wavefront then counts itself in at its group's counter;
//                     the last one publishes the group (T > 0) or finishes it
//                     (T == 0: the greedy accept step; row statistics: the
//                     row's max and sum).
//  residual blocks    (T > 0) sit a few groups after their group's statistics
//                     blocks, so they usually start after it is published. A
//                     block folds the group's partials, repeats the accept step
//                     (lane i: alpha in fp64 from the two logits of draft token
//                     i, its Philox uniform; a ballot finds the first rejection
//                     k) and its wavefronts sum, in fp64, the residual
//                     max(0, p - q) of row k (or p of the bonus row) over
//                     1024-element subsegments. The group's last wavefront to
//                     finish draws the token: wave scans of the subsegment sums,
//                     then of the chosen subsegment.
// A residual block waits only for statistics blocks of lower index, which the
// in-order dispatch has already started, and its wait is bounded in time.
// Data crossing blocks moves through device-coherent (agent-scope) atomic loads
// and stores, which bypass the per-XCD L2 caches, ordered by waiting for their
// completion; no cache flush or invalidate is issued.
// Exponentials are fp32 (v_exp_f32 on one FMA); every sum and comparison that
// decides a token is fp64.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <type_traits>
#include <utility>

#include "specverify.h"

namespace {

#ifndef SPECVERIFY_STATS_UNROLL
#define SPECVERIFY_STATS_UNROLL 4
#endif
#ifndef SPECVERIFY_CHUNKS_PER_WAVE
#define SPECVERIFY_CHUNKS_PER_WAVE 16
#endif
#ifndef SPECVERIFY_LAG
#define SPECVERIFY_LAG 1024
#endif
#ifndef SPECVERIFY_BF16_SUBS
#define SPECVERIFY_BF16_SUBS 2
#endif
#ifndef SPECVERIFY_SLEEP
#define SPECVERIFY_SLEEP 2
#endif
#ifndef SPECVERIFY_SYNC_STRIDE
#define SPECVERIFY_SYNC_STRIDE 64
#endif

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kUnroll = SPECVERIFY_STATS_UNROLL;          // chunks per pipelined load group
constexpr int kChunksPerWave = SPECVERIFY_CHUNKS_PER_WAVE; // 1 KiB chunks per statistics wavefront
constexpr int kLag = SPECVERIFY_LAG;                       // groups between statistics and residual blocks
constexpr float kRUnset = -1.0e30f;                        // lane reference before the first finite value
constexpr int kSub = kWave * 16;      // elements per residual subsegment (one wavefront, 16 per lane)
constexpr int kMaxStage = 1024;       // partial slots of one group staged in LDS (20 bytes each)
constexpr uint64_t kWaitTicks = 200000000ull;  // bound on a residual block's wait: 2 s at 100 MHz
constexpr int kSleep = SPECVERIFY_SLEEP;            // s_sleep argument between polls (64 cycles each)
constexpr int kSyncStride = SPECVERIFY_SYNC_STRIDE; // words between one group's counters and the next's

enum : int { kAcc = 0, kRej = 1, kBad = 2 };
enum : int { kSample = 0, kGreedy = 1, kRows = 2 };
enum : int { kStatsBlock = 0, kResidBlock = 1 };

// --------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11). Each round maps
// (c0, c1, c2, c3) to (hi(B*c2)^c1^k0, lo(B*c2), hi(A*c0)^c3^k1, lo(A*c0)) with
// A = 0xD2511F53, B = 0xCD9E8D57; the key advances by the golden-ratio and
// sqrt(3)-1 Weyl increments between rounds.
// --------------------------------------------------------------------------
__device__ inline double philox_uniform(uint64_t seed, uint32_t b, uint32_t i, uint32_t purpose) {
    uint32_t x0 = b, x1 = i, x2 = purpose, x3 = 0u;
    uint32_t k0 = static_cast<uint32_t>(seed), k1 = static_cast<uint32_t>(seed >> 32);
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint32_t lo_a = 0xD2511F53u * x0, hi_a = __umulhi(0xD2511F53u, x0);
        const uint32_t lo_b = 0xCD9E8D57u * x2, hi_b = __umulhi(0xCD9E8D57u, x2);
        const uint32_t y0 = hi_b ^ x1 ^ k0, y2 = hi_a ^ x3 ^ k1;
        x0 = y0; x1 = lo_b; x2 = y2; x3 = lo_a;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    const uint64_t bits53 = ((static_cast<uint64_t>(x1) << 32) | x0) >> 11;
    return static_cast<double>(bits53) * 0x1.0p-53;
}

// --------------------------------------------------------------------------
// Element access
// --------------------------------------------------------------------------
template <int DT> struct ElemBytes;
template <> struct ElemBytes<SPEC_F32> { static constexpr int value = 4; };
template <> struct ElemBytes<SPEC_BF16> { static constexpr int value = 2; };

template <int DT>
__device__ inline const char* row_at(const void* base, int64_t elem) {
    return static_cast<const char*>(base) + elem * ElemBytes<DT>::value;
}

template <int DT>
__device__ inline float load_one(const char* row, int64_t j) {
    if constexpr (DT == SPEC_F32) {
        return reinterpret_cast<const float*>(row)[j];
    } else {
        return __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(row)[j]) << 16);
    }
}

// Logits are streamed exactly once by the statistics pass: 16-byte
// non-temporal loads.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ inline uint4 load_stream(const char* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// A chunk is 64 lanes x EPL elements. Vector path (rows 16-byte aligned): lane l
// holds elements [l*EPL, l*EPL+EPL) from one 16-byte load, kept raw until
// consumed. Scalar path: lane l holds elements l, l+64, l+128, l+192, converted
// at load time. Either way each lane sees its elements in ascending order.
template <int DT, bool VEC> struct Chunk {
    static constexpr int EPL = VEC ? 16 / ElemBytes<DT>::value : 4;
    static constexpr int CH = kWave * EPL;
    using Raw = typename std::conditional<VEC, uint4, float4>::type;

    __device__ static inline Raw load_full(const char* row, int64_t c, int lane) {
        if constexpr (VEC) {
            return load_stream(row + (c * CH + lane * EPL) * ElemBytes<DT>::value);
        } else {
            const int64_t j = c * CH + lane;
            return make_float4(load_one<DT>(row, j), load_one<DT>(row, j + kWave),
                               load_one<DT>(row, j + 2 * kWave), load_one<DT>(row, j + 3 * kWave));
        }
    }
    // The last load group of a piece, with no branch around its loads: a chunk
    // past c_last, and elements at or beyond V, load from a valid address of
    // chunk min(c, c_last); mask() then replaces them by -inf where the group
    // is consumed.
    __device__ static inline Raw load_clamped(const char* row, int64_t c, int64_t c_last, int lane, int32_t V) {
        const int64_t cc = c <= c_last ? c : c_last;
        if constexpr (VEC) {
            const int64_t e = cc * CH + lane * EPL;
            return load_stream(row + (e < V ? e : cc * CH) * ElemBytes<DT>::value);  // V % EPL == 0 here
        } else {
            float v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t j = cc * CH + lane + k * kWave;
                v[k] = load_one<DT>(row, j < V ? j : cc * CH);
            }
            return make_float4(v[0], v[1], v[2], v[3]);
        }
    }
    __device__ static inline Raw mask(const Raw& w, int64_t c, int64_t c_last, int lane, int32_t V) {
        const bool cin = c <= c_last;
        if constexpr (VEC) {
            const bool ok = cin && c * CH + lane * EPL < V;
            const uint32_t ninf = DT == SPEC_F32 ? 0xFF800000u : 0xFF80FF80u;
            return make_uint4(ok ? w.x : ninf, ok ? w.y : ninf, ok ? w.z : ninf, ok ? w.w : ninf);
        } else {
            const int64_t j = c * CH + lane;
            return make_float4(cin && j < V ? w.x : -INFINITY, cin && j + kWave < V ? w.y : -INFINITY,
                               cin && j + 2 * kWave < V ? w.z : -INFINITY, cin && j + 3 * kWave < V ? w.w : -INFINITY);
        }
    }
    __device__ static inline void expand(const Raw& w, float* x) {
        if constexpr (!VEC) {
            x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
        } else if constexpr (DT == SPEC_F32) {
            x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
            x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
        } else {
            x[0] = __uint_as_float(w.x << 16); x[1] = __uint_as_float(w.x & 0xFFFF0000u);
            x[2] = __uint_as_float(w.y << 16); x[3] = __uint_as_float(w.y & 0xFFFF0000u);
            x[4] = __uint_as_float(w.z << 16); x[5] = __uint_as_float(w.z & 0xFFFF0000u);
            x[6] = __uint_as_float(w.w << 16); x[7] = __uint_as_float(w.w & 0xFFFF0000u);
        }
    }
    __device__ static inline int64_t index_of(int64_t c, int lane, int v) {
        return VEC ? c * CH + lane * EPL + v : c * CH + lane + kWave * v;
    }
};

// --------------------------------------------------------------------------
// Wave and block reductions
// --------------------------------------------------------------------------
__device__ inline float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
// fp64 moves across lanes with DPP (each 32-bit half), lanes without a source
// reading 0: row_shr:n = 0x110 + n, wave_shr:1 = 0x138, row_bcast:15 = 0x142
// (lane 15 of each row into the next row), row_bcast:31 = 0x143 (lane 31 into
// rows 2 and 3). ROWS selects the 16-lane rows that receive.
template <int CTRL, int ROWS>
__device__ inline double dpp_f64(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), CTRL, ROWS, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), CTRL, ROWS, 0xF, false);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<uint32_t>(lo));
}
__device__ inline double lane_f64(double v, int l) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), l);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), l);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<uint32_t>(lo));
}
// Inclusive prefix sum over the 64 lanes (all lanes active): Hillis-Steele
// within each row of 16, then the row totals carried across rows.
__device__ inline double wave_scan_incl(double v) {
    v += dpp_f64<0x111, 0xF>(v);
    v += dpp_f64<0x112, 0xF>(v);
    v += dpp_f64<0x114, 0xF>(v);
    v += dpp_f64<0x118, 0xF>(v);
    v += dpp_f64<0x142, 0xA>(v);
    v += dpp_f64<0x143, 0xC>(v);
    return v;
}
// Sum over the 64 lanes (all lanes active), returned to every lane.
__device__ inline double wave_sum(double v) { return lane_f64(wave_scan_incl(v), kWave - 1); }

// --------------------------------------------------------------------------
// Device-coherent access. Agent-scope atomic loads and stores bypass the L2
// cache of the XCD that issues them, so what one block publishes is read
// unchanged by a block on another XCD.
// --------------------------------------------------------------------------
__device__ inline void cst(float* p, float v) {
    __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void cst(double* p, double v) {
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                       static_cast<unsigned long long>(__double_as_longlong(v)), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void cst(int32_t* p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void cst(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float cld(const float* p) {
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
}
__device__ inline double cld(const double* p) {
    return __longlong_as_double(static_cast<long long>(
        __hip_atomic_load(reinterpret_cast<unsigned long long*>(const_cast<double*>(p)), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT)));
}
__device__ inline int32_t cld(const int32_t* p) {
    return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint32_t cld(const uint32_t* p) {
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every memory operation this wavefront issued so far has completed (so its
// coherent stores are visible device-wide) before anything after this point.
__device__ inline void complete_before() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt not waited on
}
// Loads after this point are issued after everything before it has completed.
__device__ inline void after_complete() {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}
// Cross-lane exchange through LDS inside one wavefront.
__device__ inline void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Counts the calling wavefront in at a group counter once its coherent stores
// have completed. Returns true to the last of `total` arrivals, which then sees
// every earlier arrival's stores through coherent loads, and which resets the
// counter for the next call (stream order makes the reset visible to it).
__device__ inline bool arrive_last(uint32_t* cnt, uint32_t total, int lane) {
    complete_before();
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0, kWave);
    if (old + 1u != total) return false;
    after_complete();
    if (lane == 0) cst(cnt, 0u);
    return true;
}

// --------------------------------------------------------------------------
// Launch geometry and arguments
// --------------------------------------------------------------------------
struct Params {
    int32_t G;      // groups: sequences, or rows for the stand-alone statistics
    int32_t rps;    // rows per group: 2*gamma+1 (T > 0), gamma+1 (T == 0), 1 (row statistics)
    int32_t gamma;
    int32_t V;
    int32_t nchunk; // chunks per row
    int32_t cpw;    // chunks per statistics wavefront
    int32_t nw;     // statistics wavefronts per group
    int32_t sb;     // statistics blocks per group
    int32_t rb;     // residual blocks per group (0 at T == 0)
    int32_t lag;    // groups between a group's statistics blocks and its residual blocks
    int32_t maxp;   // partial slots per row (a row spans at most maxp wavefronts)
    int32_t nsub;   // residual subsegments per row
    int32_t stage;  // a group's partial slots staged in LDS, or 0 (fold from memory)
    float c32;      // log2(e)/T
    uint64_t seed;
    int64_t b_offset;
    const void* tgt;
    const void* dft;
    const int32_t* tokens;
    int32_t* out_tokens;
    int32_t* out_n;
    float* rows_max;      // row statistics outputs
    double* rows_sumexp;
    float* part_m;        // per partial slot: max of the piece
    float* part_r;        // integer reference of the piece (T > 0)
    double* part_s;       // sum of 2^(x*c - reference) (T > 0)
    int32_t* part_i;      // first index of the maximum (T == 0)
    double* sub_r;        // [G, nsub] residual mass per subsegment (t units)
    uint32_t* cnt_s;      // [G] statistics blocks counted in
    uint32_t* cnt_r;      // [G] residual blocks counted in (T > 0)
    uint32_t* err;        // sticky: a residual block's wait ran out
    float* dbg_row_max;
    double* dbg_row_sumexp;
    double* dbg_p;
    double* dbg_q;
    double* dbg_z;
    int32_t* dbg_argmax;
};

// Grid order: groups [0, lag) contribute their statistics blocks; each group
// j in [lag, G) then contributes its statistics blocks followed by the
// residual blocks of group j - lag; the residual blocks of the last lag groups
// close the grid. A group's residual blocks thus always follow all of its
// statistics blocks.
__device__ inline void decode_block(const Params& P, uint32_t x, int& kind, uint32_t& g, uint32_t& idx) {
    const uint32_t S = static_cast<uint32_t>(P.sb), R = static_cast<uint32_t>(P.rb);
    const uint32_t D = static_cast<uint32_t>(P.lag), G = static_cast<uint32_t>(P.G);
    const uint32_t head = D * S;
    if (x < head) {
        kind = kStatsBlock;
        g = x / S;
        idx = x - g * S;
        return;
    }
    x -= head;
    const uint32_t per = S + R;
    const uint32_t mid = (G - D) * per;
    if (x < mid) {
        const uint32_t t = x / per, o = x - t * per;
        if (o < S) {
            kind = kStatsBlock;
            g = D + t;
            idx = o;
        } else {
            kind = kResidBlock;
            g = t;
            idx = o - S;
        }
        return;
    }
    x -= mid;  // only reached when R > 0
    kind = kResidBlock;
    const uint32_t t = x / R;
    g = (G - D) + t;
    idx = x - t * R;
}

// Row j of group g: target rows 0..gamma, then (T > 0) draft rows 0..gamma-1.
template <int DT, int MODE>
__device__ inline const char* group_row(const Params& P, uint32_t g, uint32_t j) {
    if constexpr (MODE == kRows) {
        return row_at<DT>(P.tgt, static_cast<int64_t>(g) * P.V);
    } else {
        const uint32_t nt = static_cast<uint32_t>(P.gamma) + 1u;
        if (MODE == kGreedy || j < nt) return row_at<DT>(P.tgt, (static_cast<int64_t>(g) * nt + j) * P.V);
        return row_at<DT>(P.dft, (static_cast<int64_t>(g) * P.gamma + (j - nt)) * P.V);
    }
}

struct SoftLane {
    float m;
    float R;
    double S;
    __device__ inline void init() { m = -INFINITY; R = kRUnset; S = 0.0; }
};
struct ArgLane {
    float best;
    int32_t at;
    bool nan;
    __device__ inline void init() { best = -INFINITY; at = INT32_MAX; nan = false; }
};

__device__ inline double rebase(double S, float R, float Rto) {
    return S == 0.0 ? 0.0 : ldexp(S, static_cast<int>(fmaxf(R - Rto, -1100.0f)));
}

// Sum of 2^(fl(x*c - R)) over a load group, expanding each 16-byte load as it
// is consumed (the raw loads stay live for the rare redo).
template <int DT, bool VEC, int N>
__device__ inline void group_sum(const typename Chunk<DT, VEC>::Raw* raw, float c, float R, float& gmax,
                                 float& acc) {
    using C = Chunk<DT, VEC>;
    float a0 = 0.0f, a1 = 0.0f, mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < N; ++u) {
        float x[C::EPL];
        C::expand(raw[u], x);
#pragma unroll
        for (int v = 0; v < C::EPL; ++v) {
            mx = fmaxf(mx, x[v]);
            const float e = __builtin_amdgcn_exp2f(fmaf(x[v], c, -R));
            if (v & 1) a1 += e;
            else a0 += e;
        }
    }
    gmax = mx;
    acc = a0 + a1;
}

template <int DT, bool VEC, int N>
__device__ inline float group_max(const typename Chunk<DT, VEC>::Raw* raw) {
    using C = Chunk<DT, VEC>;
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < N; ++u) {
        float x[C::EPL];
        C::expand(raw[u], x);
#pragma unroll
        for (int v = 0; v < C::EPL; ++v) mx = fmaxf(mx, x[v]);
    }
    return mx;
}

template <int DT, bool VEC, int N>
__device__ inline void consume_group(SoftLane& s, const typename Chunk<DT, VEC>::Raw* raw, int64_t, int,
                                     float c) {
    if (s.R == kRUnset) {  // no reference yet: take it from the wave's max of this group first
        const float mx = wave_max(group_max<DT, VEC, N>(raw));
        if (mx * c > kRUnset + 1.0f) {
            const float Rn = ceilf(mx * c);
            if (Rn < 3.0e38f) s.R = Rn;
        }
    }
    float gmax, acc;
    group_sum<DT, VEC, N>(raw, c, s.R, gmax, acc);
    if (__any(gmax * c > s.R + 1.0f)) {  // rare: a new maximum well above the wave's reference
        const float Rn = ceilf(wave_max(gmax) * c);
        if (!(Rn < 3.0e38f)) {  // +inf logit (or an overflowing one): the row is unusable
            s.S = NAN;
            acc = 0.0f;
        } else {
            if (s.R > kRUnset) s.S = ldexp(s.S, static_cast<int>(fmaxf(s.R - Rn, -1100.0f)));
            s.R = Rn;
            float unused;
            group_sum<DT, VEC, N>(raw, c, s.R, unused, acc);
        }
    }
    s.m = fmaxf(s.m, gmax);
    s.S += static_cast<double>(acc);
}

template <int DT, bool VEC, int N>
__device__ inline void consume_group(ArgLane& s, const typename Chunk<DT, VEC>::Raw* raw, int64_t c0,
                                     int lane, float) {
    using C = Chunk<DT, VEC>;
#pragma unroll
    for (int u = 0; u < N; ++u) {
        float x[C::EPL];
        C::expand(raw[u], x);
#pragma unroll
        for (int v = 0; v < C::EPL; ++v) {
            s.nan |= (x[v] != x[v]);
            if (x[v] > s.best) { s.best = x[v]; s.at = static_cast<int32_t>(C::index_of(c0 + u, lane, v)); }
        }
    }
}


// One row piece's partial, handed through LDS to the block's last wavefront,
// which writes the block's pieces to memory.
struct Piece {
    int64_t slot;  // (g*rps + j)*maxp + k
    double s;      // sum of 2^(x*c - r) (T > 0)
    float m;       // max of the piece
    float r;       // integer reference (T > 0)
    int32_t i;     // first index of the maximum (T == 0)
    int32_t npad;  // neutral slots after this one (the piece that ends its row)
};
constexpr int kMaxPieces = 4;  // row pieces per wavefront (the host keeps cpw <= 3 rows of chunks)
struct BlockPieces {
    Piece p[kWavesPerBlock][kMaxPieces];
    int32_t n[kWavesPerBlock];
    uint32_t done;
};

// Statistics of one wavefront's chunk range [wl*cpw, (wl+1)*cpw) of group g's
// concatenated rows: one partial per row piece, for slot (g*rps + j)*maxp + k,
// k = wl minus the first wavefront touching row j. The piece that ends a row
// also covers the row's unused slots (a row spans maxp - 1 or maxp
// wavefronts), which are written with neutral values, so folds read every
// slot. Returns the number of pieces placed in `out` (lane 0 writes them).
template <int DT, bool VEC, int MODE>
__device__ inline int stats_wave(const Params& P, uint32_t g, uint32_t wl, int lane, Piece* out) {
    int npieces = 0;
    using C = Chunk<DT, VEC>;
    using Raw = typename C::Raw;
    using Lane = typename std::conditional<MODE == kGreedy, ArgLane, SoftLane>::type;
    const float c = P.c32;
    const uint32_t nchunk = static_cast<uint32_t>(P.nchunk), cpw = static_cast<uint32_t>(P.cpw);
    const uint32_t total = static_cast<uint32_t>(P.rps) * nchunk;
    uint32_t cc = wl * cpw;
    const uint32_t c_end = cc + cpw < total ? cc + cpw : total;
    uint32_t j = cc / nchunk;
    uint32_t first = j * nchunk;
    int32_t k = static_cast<int32_t>(wl - first / cpw);
    while (cc < c_end) {
        const uint32_t ce = first + nchunk < c_end ? first + nchunk : c_end;
        const char* row = group_row<DT, MODE>(P, g, j);
        const int64_t c0 = cc - first, c1 = ce - first;  // this piece: chunks [c0, c1) of row j
        Lane st;
        st.init();
        // load groups of kUnroll chunks. Every group but the last lies wholly in
        // the piece and in the row; the last may run past c1 or V (clamped
        // loads, masked where consumed). Two register buffers are used in turn:
        // one group's loads are in flight while the other is consumed, and no
        // load sits under a branch, so each wait covers exactly one group.
        const int64_t ng = (c1 - c0 + kUnroll - 1) / kUnroll;
        const int64_t c_last = c1 - 1;
        Raw qa[kUnroll], qb[kUnroll];
        // (a scheduling barrier after each group keeps its loads ahead of the
        // consumption of the previous group)
        auto load = [&](Raw* q, int64_t gi) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) q[u] = C::load_full(row, c0 + gi * kUnroll + u, lane);
            __builtin_amdgcn_sched_barrier(0);
        };
        auto load_last = [&](Raw* q, int64_t gi) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) q[u] = C::load_clamped(row, c0 + gi * kUnroll + u, c_last, lane, P.V);
            __builtin_amdgcn_sched_barrier(0);
        };
        auto eat = [&](const Raw* q, int64_t gi) { consume_group<DT, VEC, kUnroll>(st, q, c0 + gi * kUnroll, lane, c); };
        auto eat_last = [&](Raw* q, int64_t gi) {
            const int64_t cg = c0 + gi * kUnroll;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) q[u] = C::mask(q[u], cg + u, c_last, lane, P.V);
            eat(q, gi);
        };
        if (ng == 1) {
            load_last(qa, 0);
            eat_last(qa, 0);
        } else {
            load(qa, 0);
            int64_t gi = 1;  // next group to load; qa holds group gi - 1
            for (; gi + 2 < ng; gi += 2) {  // groups gi and gi + 1 are not the last
                load(qb, gi);
                eat(qa, gi - 1);
                load(qa, gi + 1);
                eat(qb, gi);
            }
            if (gi + 1 == ng) {  // gi is the last group
                load_last(qb, gi);
                eat(qa, gi - 1);
                eat_last(qb, gi);
            } else {             // gi, then the last group gi + 1
                load(qb, gi);
                eat(qa, gi - 1);
                load_last(qa, gi + 1);
                eat(qb, gi);
                eat_last(qa, gi + 1);
            }
        }
        Piece pc;
        pc.slot = (static_cast<int64_t>(g) * P.rps + j) * P.maxp + k;
        pc.npad = ce == first + nchunk ? P.maxp - 1 - k : 0;
        if constexpr (MODE == kGreedy) {
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {  // (value desc, index asc) across the wave
                const float ob = __shfl_xor(st.best, o, kWave);
                const int32_t oa = __shfl_xor(st.at, o, kWave);
                if (ob > st.best || (ob == st.best && oa < st.at)) {
                    st.best = ob;
                    st.at = oa;
                }
            }
            pc.m = __ballot(st.nan) != 0 ? NAN : st.best;
            pc.i = st.at;
            pc.r = 0.0f;
            pc.s = 0.0;
        } else {
            pc.m = wave_max(st.m);
            pc.r = st.R;  // shared by the wave
            pc.s = wave_sum(st.S);
            pc.i = 0;
        }
        if (lane == 0 && npieces < kMaxPieces) out[npieces] = pc;
        ++npieces;
        cc = ce;
        ++j;  // a later piece of this wave starts its row: slot 0
        first += nchunk;
        k = 0;
    }
    return npieces;
}

// The block's last statistics wavefront writes every piece of the block (and
// the neutral slots after row-ending pieces) with coherent stores: lane e
// takes piece e % kMaxPieces of wavefront e / kMaxPieces.
template <int MODE>
__device__ inline void write_pieces(const Params& P, const BlockPieces& bp, int nwaves, int lane) {
    const int ww = lane / kMaxPieces, q = lane - ww * kMaxPieces;
    if (ww >= nwaves || q >= bp.n[ww]) return;
    const Piece pc = bp.p[ww][q];
    if constexpr (MODE == kGreedy) {
        cst(P.part_m + pc.slot, pc.m);
        cst(P.part_i + pc.slot, pc.i);
        for (int t = 1; t <= pc.npad; ++t) {
            cst(P.part_m + pc.slot + t, -INFINITY);
            cst(P.part_i + pc.slot + t, INT32_MAX);
        }
    } else {
        cst(P.part_m + pc.slot, pc.m);
        cst(P.part_r + pc.slot, pc.r);
        cst(P.part_s + pc.slot, pc.s);
        for (int t = 1; t <= pc.npad; ++t) {
            cst(P.part_m + pc.slot + t, -INFINITY);
            cst(P.part_r + pc.slot + t, kRUnset);
            cst(P.part_s + pc.slot + t, 0.0);
        }
    }
}

// --------------------------------------------------------------------------
// Folding partials. A row's partials (M_p, R_p, S_p) combine exactly with
// ldexp onto the largest reference R; the result is rebased once to the row
// max: S * 2^(R - M*c), the exponent formed exactly in fp64. The argmax
// partials combine as (value desc, index asc); any NaN marks the row.
// --------------------------------------------------------------------------
struct RowStat {
    float m;
    int32_t arg;
    double s;
};

__device__ inline bool usable(float M, double S) { return isfinite(M) && isfinite(S) && S > 0.0; }

// One thread folds one row's np slots, staged in LDS, in slot order.
template <bool GREEDY>
__device__ inline RowStat fold_slots(int np, const float* pm, const float* pr, const double* ps, const int32_t* pi,
                                     float c32) {
    RowStat o;
    if constexpr (GREEDY) {
        float best = -INFINITY;
        int32_t arg = INT32_MAX;
        bool nan = false;
        for (int k = 0; k < np; ++k) {
            const float v = pm[k];
            const int32_t a = pi[k];
            nan |= (v != v);
            if (v > best || (v == best && a < arg)) {
                best = v;
                arg = a;
            }
        }
        o.m = nan ? NAN : best;
        o.arg = arg;
        o.s = 1.0;
    } else {
        float M = -INFINITY, R = kRUnset;
        for (int k = 0; k < np; ++k) {
            M = fmaxf(M, pm[k]);
            R = fmaxf(R, pr[k]);
        }
        double acc = 0.0;
        for (int k = 0; k < np; ++k) acc += rebase(ps[k], pr[k], R);
        o.m = M;
        o.arg = 0;
        o.s = acc * exp2(static_cast<double>(R) - static_cast<double>(M) * static_cast<double>(c32));
    }
    return o;
}

// The same fold straight from memory (coherent loads, eight slots in flight),
// for groups whose slots do not fit the LDS stage. The running sum is rebased
// by powers of two as the reference grows, which gives the staged fold's value.
template <bool GREEDY>
__device__ inline RowStat fold_slots_mem(const Params& P, int64_t base) {
    constexpr int kB = 8;
    const int np = P.maxp;
    RowStat o;
    if constexpr (GREEDY) {
        float best = -INFINITY;
        int32_t arg = INT32_MAX;
        bool nan = false;
        for (int k0 = 0; k0 < np; k0 += kB) {
            float v[kB];
            int32_t a[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                v[u] = k0 + u < np ? cld(P.part_m + base + k0 + u) : -INFINITY;
                a[u] = k0 + u < np ? cld(P.part_i + base + k0 + u) : INT32_MAX;
            }
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                nan |= (v[u] != v[u]);
                if (v[u] > best || (v[u] == best && a[u] < arg)) {
                    best = v[u];
                    arg = a[u];
                }
            }
        }
        o.m = nan ? NAN : best;
        o.arg = arg;
        o.s = 1.0;
    } else {
        float M = -INFINITY, R = kRUnset;
        double S = 0.0;
        for (int k0 = 0; k0 < np; k0 += kB) {
            float m[kB], r[kB];
            double s[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                const bool in = k0 + u < np;
                m[u] = in ? cld(P.part_m + base + k0 + u) : -INFINITY;
                r[u] = in ? cld(P.part_r + base + k0 + u) : kRUnset;
                s[u] = in ? cld(P.part_s + base + k0 + u) : 0.0;
            }
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                const float Rn = fmaxf(R, r[u]);
                S = rebase(S, R, Rn) + rebase(s[u], r[u], Rn);
                R = Rn;
                M = fmaxf(M, m[u]);
            }
        }
        o.m = M;
        o.arg = 0;
        o.s = S * exp2(static_cast<double>(R) - static_cast<double>(M) * static_cast<double>(P.c32));
    }
    return o;
}

// One wavefront folds one row (the stand-alone row statistics): lane k takes
// slots k, k+64, ...; butterfly reductions combine the lanes.
__device__ inline RowStat fold_row_wave(const Params& P, int64_t base, int lane) {
    float M = -INFINITY, R = kRUnset;
    double S = 0.0;
    for (int k = lane; k < P.maxp; k += kWave) {
        const float mk = cld(P.part_m + base + k), rk = cld(P.part_r + base + k);
        const double sk = cld(P.part_s + base + k);
        const float Rn = fmaxf(R, rk);
        S = rebase(S, R, Rn) + rebase(sk, rk, Rn);
        R = Rn;
        M = fmaxf(M, mk);
    }
    const float Mw = wave_max(M), Rw = wave_max(R);
    const double Sw = wave_sum(rebase(S, R, Rw));
    RowStat o;
    o.m = Mw;
    o.arg = 0;
    o.s = Sw * exp2(static_cast<double>(Rw) - static_cast<double>(Mw) * static_cast<double>(P.c32));
    return o;
}

// Running fold state of a set of partials: soft (max m, reference r, sum s of
// 2^(x*c - r)) or argmax (best value, its first index, any NaN).
struct Fold {
    float m, r;
    double s;
    int32_t arg;
    bool nan;
};
__device__ inline Fold fold_init() { return Fold{-INFINITY, kRUnset, 0.0, INT32_MAX, false}; }
template <bool GREEDY>
__device__ inline void fold_add(Fold& f, float m, float r, double s, int32_t arg) {
    if constexpr (GREEDY) {
        f.nan |= (m != m);
        if (m > f.m || (m == f.m && arg < f.arg)) {
            f.m = m;
            f.arg = arg;
        }
    } else {
        const float rn = fmaxf(f.r, r);
        f.s = rebase(f.s, f.r, rn) + rebase(s, r, rn);
        f.r = rn;
        f.m = fmaxf(f.m, m);
    }
}

// The rps rows of group g folded into rs[0, rps) (LDS) by NT threads (a block,
// or one wavefront). If the group's rps*maxp slots fit the stage, each thread
// loads its share of them at once into LDS (one round trip), then q threads
// per row (a power of two up to 16, q*rps <= NT) fold strided slots and
// combine with butterfly shuffles; otherwise thread j folds row j from memory.
template <bool GREEDY, int NT>
__device__ inline void merge_group(const Params& P, uint32_t g, char* dyn, RowStat* rs) {
    constexpr int kPer = (kMaxStage + NT - 1) / NT;  // staged slots per thread
    const int maxp = P.maxp, nrows = P.rps;
    const int slots = nrows * maxp;
    const int tid = NT == kWave ? static_cast<int>(threadIdx.x & (kWave - 1)) : static_cast<int>(threadIdx.x);
    const int64_t base = static_cast<int64_t>(g) * slots;
    auto sync = [] {
        if constexpr (NT == kWave) wave_lds_sync();
        else __syncthreads();
    };
    if (P.stage > 0) {
        const int cap = P.stage;
        double* ls = reinterpret_cast<double*>(dyn);
        float* lm = reinterpret_cast<float*>(ls + cap);
        float* lr = lm + cap;
        int32_t* li = reinterpret_cast<int32_t*>(lr + cap);
        float vm[kPer], vr[kPer];
        double vs[kPer];
        int32_t vi[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int t = u * NT + tid;
            if (t < slots) {
                vm[u] = cld(P.part_m + base + t);
                if constexpr (GREEDY) {
                    vi[u] = cld(P.part_i + base + t);
                } else {
                    vr[u] = cld(P.part_r + base + t);
                    vs[u] = cld(P.part_s + base + t);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int t = u * NT + tid;
            if (t < slots) {
                lm[t] = vm[u];
                if constexpr (GREEDY) {
                    li[t] = vi[u];
                } else {
                    lr[t] = vr[u];
                    ls[t] = vs[u];
                }
            }
        }
        sync();
        int q = 1;
        while (q < 16 && 2 * q * nrows <= NT) q *= 2;
        const int rows_per_pass = NT / q;
        for (int j0 = 0; j0 < nrows; j0 += rows_per_pass) {
            const int j = j0 + tid / q, part = tid % q;
            Fold f = fold_init();
            if (j < nrows)
                for (int k = part; k < maxp; k += q) {
                    const int t = j * maxp + k;
                    fold_add<GREEDY>(f, lm[t], GREEDY ? 0.0f : lr[t], GREEDY ? 0.0 : ls[t], GREEDY ? li[t] : 0);
                }
            for (int o = q / 2; o > 0; o >>= 1) {  // combine the q threads of the row (same wavefront)
                const float om = __shfl_xor(f.m, o, kWave);
                if constexpr (GREEDY) {
                    const int32_t oa = __shfl_xor(f.arg, o, kWave);
                    const bool on = __shfl_xor(f.nan ? 1 : 0, o, kWave) != 0;
                    fold_add<true>(f, om, 0.0f, 0.0, oa);
                    f.nan |= on;
                } else {
                    const float orr = __shfl_xor(f.r, o, kWave);
                    const double os = __shfl_xor(f.s, o, kWave);
                    fold_add<false>(f, om, orr, os, 0);
                }
            }
            if (j < nrows && part == 0) {
                RowStat o;
                o.m = GREEDY && f.nan ? NAN : f.m;
                o.arg = GREEDY ? f.arg : 0;
                o.s = GREEDY ? 1.0
                             : f.s * exp2(static_cast<double>(f.r) - static_cast<double>(f.m) * static_cast<double>(P.c32));
                rs[j] = o;
            }
        }
    } else {
        for (int j = tid; j < nrows; j += NT) rs[j] = fold_slots_mem<GREEDY>(P, base + static_cast<int64_t>(j) * maxp);
    }
    sync();
}

// What the residual sums and the draw need about the row a sequence resamples.
struct SeqInfo {
    int32_t k;       // emitted position (0..gamma), -1 = invalid sequence
    float mcp, mcq;  // fl(max*c) of the target row k / draft row k
    int32_t has_q;   // 0 at the bonus row (k == gamma)
    double rho;      // scale_q / scale_p
    double scale_p;  // 2^(mcp - max_p*c) / S_p: probability per t unit
};

// The residual constants of a row pair from its folded stats (max m, sum S).
__device__ inline SeqInfo seq_info(int k, bool has_q, float mp, double sp, float mq, double sq, float c32) {
    SeqInfo si;
    const double c = static_cast<double>(c32);
    si.k = k;
    si.has_q = has_q ? 1 : 0;
    si.mcp = mp * c32;
    si.scale_p = exp2(static_cast<double>(si.mcp) - static_cast<double>(mp) * c) / sp;
    si.mcq = has_q ? mq * c32 : 0.0f;
    si.rho = has_q ? exp2(static_cast<double>(si.mcq) - static_cast<double>(mq) * c) / sq / si.scale_p : 0.0;
    return si;
}

// --------------------------------------------------------------------------
// The accept step, by one wavefront after the group's rows are folded into rs
// (target rows 0..gamma, then draft rows at T > 0): lane i takes draft token
// i, forms alpha in fp64 (greedy: compares the token with the row's argmax),
// draws its Philox uniform, and a ballot finds the first rejection k. With
// `emit` it writes k, the accepted tokens and the -1 padding (greedy also the
// emitted argmax; the sampled token at k is left to the draw) and the debug
// values. Returns the sequence record the residual needs.
// --------------------------------------------------------------------------
template <bool GREEDY>
__device__ inline SeqInfo accept_wave(const Params& P, uint32_t g, const RowStat* rs, int32_t x, float lt, float ld,
                                      bool emit) {
    const int32_t gamma = P.gamma, V = P.V;
    const int nt = gamma + 1;
    const int i = static_cast<int>(threadIdx.x & (kWave - 1));
    const int64_t b = g;
    const int64_t R = 2 * gamma + 1;
    const bool tok_ok = x >= 0 && x < V;
    int status = kAcc;
    float mt = NAN, md = NAN;
    double st = NAN, sd = NAN;
    bool ut = false;
    int32_t amax = -1;
    if (i <= gamma) {
        const RowStat t = rs[i];
        mt = t.m;
        if (emit && P.dbg_row_max) P.dbg_row_max[b * R + i] = mt;
        if constexpr (GREEDY) {
            amax = t.arg;
            ut = isfinite(mt);
            if (emit && P.dbg_argmax) P.dbg_argmax[b * nt + i] = amax;
        } else {
            st = t.s;
            ut = usable(mt, st);
            if (emit && P.dbg_row_sumexp) P.dbg_row_sumexp[b * R + i] = st;
        }
    }
    if (i < gamma) {
        if constexpr (GREEDY) {
            status = (!ut || !tok_ok) ? kBad : (x == amax ? kAcc : kRej);
        } else {
            const RowStat dr = rs[nt + i];
            md = dr.m;
            sd = dr.s;
            const bool ud = usable(md, sd);
            if (emit && P.dbg_row_max) P.dbg_row_max[b * R + nt + i] = md;
            if (emit && P.dbg_row_sumexp) P.dbg_row_sumexp[b * R + nt + i] = sd;
            double p = NAN, q = NAN;
            if (!ut || !ud || !tok_ok) {
                status = kBad;
            } else {
                const double c = static_cast<double>(P.c32);
                p = exp2((static_cast<double>(lt) - static_cast<double>(mt)) * c) / st;
                q = exp2((static_cast<double>(ld) - static_cast<double>(md)) * c) / sd;
                const double alpha = p == 0.0 ? 0.0 : (q == 0.0 ? 1.0 : fmin(1.0, p / q));
                const double u = philox_uniform(P.seed, static_cast<uint32_t>(b + P.b_offset),
                                                static_cast<uint32_t>(i), 0u);
                status = u < alpha ? kAcc : kRej;
            }
            if (emit && P.dbg_p) P.dbg_p[b * gamma + i] = p;
            if (emit && P.dbg_q) P.dbg_q[b * gamma + i] = q;
        }
    }
    SeqInfo mine{};
    if constexpr (!GREEDY) {
        if (i <= gamma) mine = seq_info(i, i < gamma, mt, st, md, sd, P.c32);
    }
    const uint64_t stop = __ballot(i < gamma && status != kAcc);
    const int f = stop ? __ffsll(static_cast<unsigned long long>(stop)) - 1 : gamma;
    const int fstat = __shfl(status, f, kWave);
    const bool bonus_ok = __shfl(ut ? 1 : 0, gamma, kWave) != 0;
    const bool invalid = f < gamma ? (fstat == kBad) : !bonus_ok;
    const int k = invalid ? -1 : f;
    if (emit) {
        if (i <= gamma) {
            int32_t o = -1;
            bool write = true;
            if (!invalid) {
                if (i < k) o = x;
                else if (i == k) {
                    if constexpr (GREEDY) o = amax;
                    else write = false;
                }
            }
            if (write) cst(P.out_tokens + b * nt + i, o);
        }
        if (i == 0) {
            cst(P.out_n + b, k);
            if (!GREEDY && invalid && P.dbg_z) P.dbg_z[b] = NAN;
        }
    }
    SeqInfo si;
    si.k = -1; si.mcp = 0.0f; si.mcq = 0.0f; si.has_q = 0; si.rho = 0.0; si.scale_p = 0.0;
    if constexpr (!GREEDY) {
        // lane k holds the constants of row k (every lane formed its own
        // before the ballot); broadcast them
        const int src = invalid ? 0 : k;
        const float mcp = __shfl(mine.mcp, src, kWave), mcq = __shfl(mine.mcq, src, kWave);
        const double rho = __shfl(mine.rho, src, kWave), scale_p = __shfl(mine.scale_p, src, kWave);
        if (!invalid) {
            si.k = k;
            si.has_q = k < gamma ? 1 : 0;
            si.mcp = mcp;
            si.mcq = mcq;
            si.rho = rho;
            si.scale_p = scale_p;
        }
    }
    return si;
}

// --------------------------------------------------------------------------
// Residual in t units. With e_j = 2^(fl(x_j*c - mc)) for the target (p) and
// draft (q) rows, p_j = e_pj * scale_p and q_j = e_qj * scale_q (scale =
// 2^(mc - m*c)/S). Then max(0, p_j - q_j) = scale_p * t_j with
// t_j = max(0, e_pj - rho*e_qj), rho = scale_q/scale_p. t_j is formed in fp32
// with rho split into an fp32 pair (hi + lo, two FMAs), so the product keeps
// about 48 bits; the sums over elements are fp64. The inverse-CDF draw is
// invariant to the common factor; at the bonus row t_j = e_pj.
// --------------------------------------------------------------------------
struct ResidRow {
    const char* prow;
    const char* qrow;  // nullptr at the bonus row
    float mcp, mcq;
    float rhi, rlo;    // rho = rhi + rlo
};

template <int DT>
__device__ inline ResidRow resid_row(const Params& P, const SeqInfo& s, uint32_t g) {
    ResidRow rr;
    rr.prow = group_row<DT, kSample>(P, g, static_cast<uint32_t>(s.k));
    rr.qrow = s.has_q ? group_row<DT, kSample>(P, g, static_cast<uint32_t>(P.gamma + 1 + s.k)) : nullptr;
    rr.mcp = s.mcp;
    rr.mcq = s.mcq;
    rr.rhi = static_cast<float>(s.rho);
    rr.rlo = static_cast<float>(s.rho - static_cast<double>(rr.rhi));
    return rr;
}

// One element's residual mass in t units (its p mass when !has_q). Masked
// elements carry -inf logits on both rows and give 0.
__device__ inline float resid_t(float xp, float xq, bool has_q, float c32, const ResidRow& rr) {
    const float ep = __builtin_amdgcn_exp2f(fmaf(xp, c32, -rr.mcp));
    if (!has_q) return ep;
    const float eq = __builtin_amdgcn_exp2f(fmaf(xq, c32, -rr.mcq));
    return fmaxf(0.0f, fmaf(-eq, rr.rlo, fmaf(-eq, rr.rhi, ep)));
}

// Residual subsegments one wavefront keeps in flight: 64 VGPRs of raw 16-byte
// loads (vector path), one subsegment on the scalar path.
template <int DT, bool VEC>
__host__ __device__ constexpr int subs_per_wave() { return VEC ? (DT == SPEC_BF16 ? SPECVERIFY_BF16_SUBS : 2) : 1; }

// Raw loads of one lane's 16 elements of a subsegment (vector path): each
// 16-byte load is taken only if it starts below V, which puts it wholly inside
// the row (V % EPL == 0 there); the rest read as -inf (no mass).
template <int DT>
struct SubRaw {
    static constexpr int EPL = 16 / ElemBytes<DT>::value;
    static constexpr int NV = 16 / EPL;
    uint4 p[NV], q[NV];
    __device__ inline void load(const ResidRow& rr, bool has_q, int64_t j0, int32_t V) {
        const uint32_t ninf = DT == SPEC_F32 ? 0xFF800000u : 0xFF80FF80u;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int64_t j = j0 + u * EPL;
            const bool in = j < V;
            p[u] = in ? *reinterpret_cast<const uint4*>(rr.prow + j * ElemBytes<DT>::value)
                      : make_uint4(ninf, ninf, ninf, ninf);
            q[u] = in && has_q ? *reinterpret_cast<const uint4*>(rr.qrow + j * ElemBytes<DT>::value)
                               : make_uint4(ninf, ninf, ninf, ninf);
        }
    }
};

// The 16 elements of lane `lane` in subsegment i: j0 = i*kSub + 16*lane, ...
// (p row; q row when has_q). Vector path: 16-byte loads, each taken only if it
// starts below V, which puts it wholly inside the row (V % EPL == 0 there).
// Elements at or beyond V read as -inf (no mass).
template <int DT, bool VEC>
__device__ inline void load_sub(const ResidRow& rr, bool has_q, int64_t j0, int32_t V, float* xp, float* xq) {
    if constexpr (VEC) {
        constexpr int EPL = 16 / ElemBytes<DT>::value;
        constexpr int NV = 16 / EPL;
        uint4 wp[NV], wq[NV];
        const uint32_t ninf = DT == SPEC_F32 ? 0xFF800000u : 0xFF80FF80u;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int64_t j = j0 + u * EPL;
            const bool in = j < V;
            wp[u] = in ? *reinterpret_cast<const uint4*>(rr.prow + j * ElemBytes<DT>::value)
                       : make_uint4(ninf, ninf, ninf, ninf);
            wq[u] = in && has_q ? *reinterpret_cast<const uint4*>(rr.qrow + j * ElemBytes<DT>::value)
                                : make_uint4(ninf, ninf, ninf, ninf);
        }
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            Chunk<DT, true>::expand(wp[u], xp + u * EPL);
            Chunk<DT, true>::expand(wq[u], xq + u * EPL);
        }
    } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const bool in = j0 + v < V;
            xp[v] = in ? load_one<DT>(rr.prow, j0 + v) : -INFINITY;
            xq[v] = in && has_q ? load_one<DT>(rr.qrow, j0 + v) : -INFINITY;
        }
    }
}

// --------------------------------------------------------------------------
// The draw, by the group's last residual wavefront: wave scans of the
// subsegment masses give Z and the subsegment holding u*Z; a scan over that
// subsegment's 1024 elements (16 per lane, in registers) gives the first index
// whose cumulative mass exceeds u*Z. If rounding leaves no residual mass at a
// rejected row the draw is made from p_k instead (its masses come from the
// same pass).
// --------------------------------------------------------------------------
__device__ inline double wave_scan(double v, int) { return wave_scan_incl(v); }
// The value of lane l - 1 (0 in lane 0).
__device__ inline double lane_before(double v) { return dpp_f64<0x138, 0xF>(v); }

// Total of m[0, n) in the order the search below accumulates it.
__device__ inline double scan_total(const double* m, int32_t n, int lane) {
    double base = 0.0;
    for (int32_t t0 = 0; t0 < n; t0 += kWave) {
        const double v = t0 + lane < n ? cld(m + t0 + lane) : 0.0;
        base += lane_f64(wave_scan(v, lane), kWave - 1);
    }
    return base;
}

// First index i in [0, n) whose cumulative mass exceeds t, and the mass before
// it; if rounding leaves none, the last index with mass.
__device__ inline int32_t scan_find(const double* m, int32_t n, double t, int lane, double& before) {
    double base = 0.0;
    int32_t last = -1;
    double last_before = 0.0;
    for (int32_t t0 = 0; t0 < n; t0 += kWave) {
        const double v = t0 + lane < n ? cld(m + t0 + lane) : 0.0;
        const double incl = base + wave_scan(v, lane);
        const double prev = lane_before(incl);
        const double excl = lane == 0 ? base : prev;
        const uint64_t hit = __ballot(v > 0.0 && excl <= t && t < incl);
        if (hit) {
            const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
            before = __shfl(excl, l, kWave);
            return t0 + l;
        }
        const uint64_t mass = __ballot(v > 0.0);
        if (mass) {
            const int l = 63 - __clzll(static_cast<unsigned long long>(mass));
            last = t0 + l;
            last_before = __shfl(excl, l, kWave);
        }
        base = lane_f64(incl, kWave - 1);
    }
    before = last_before;
    return last;
}

// The same two steps on up to kDrawTiles*64 masses held in registers (one
// load round trip); the totals and prefix sums are formed exactly as above.
constexpr int kDrawTiles = 4;

__device__ inline double regs_scan(const double* v, double* incl, int lane) {
    double base = 0.0;
#pragma unroll
    for (int t = 0; t < kDrawTiles; ++t) {
        incl[t] = base + wave_scan(v[t], lane);
        base = lane_f64(incl[t], kWave - 1);
    }
    return base;
}

__device__ inline int32_t regs_find(const double* v, const double* incl, double t, int lane, double& before) {
    int32_t last = -1;
    double last_before = 0.0;
#pragma unroll
    for (int k = 0; k < kDrawTiles; ++k) {
        const double prev = lane_before(incl[k]);
        const double base = k == 0 ? 0.0 : lane_f64(incl[k - 1], kWave - 1);
        const double excl = lane == 0 ? base : prev;
        const uint64_t hit = __ballot(v[k] > 0.0 && excl <= t && t < incl[k]);
        if (hit) {
            const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
            before = __shfl(excl, l, kWave);
            return k * kWave + l;
        }
        const uint64_t mass = __ballot(v[k] > 0.0);
        if (mass) {
            const int l = 63 - __clzll(static_cast<unsigned long long>(mass));
            last = k * kWave + l;
            last_before = __shfl(excl, l, kWave);
        }
    }
    before = last_before;
    return last;
}

// p masses per subsegment of the target row k, written over the residual
// masses (only when those are all zero, so nothing is lost): the draw's
// fallback from p_k, one wavefront, never on the common path.
template <int DT, bool VEC>
__device__ inline void p_masses(const Params& P, uint32_t g, const SeqInfo& in, double* sr, int lane) {
    const ResidRow rr = resid_row<DT>(P, in, g);
    for (int32_t i = 0; i < P.nsub; ++i) {
        float xp[16], xq[16];
        load_sub<DT, VEC>(rr, false, static_cast<int64_t>(i) * kSub + 16 * lane, P.V, xp, xq);
        double t = 0.0;
        for (int v = 0; v < 16; ++v) t += static_cast<double>(resid_t(xp[v], xq[v], false, P.c32, rr));
        t = wave_sum(t);
        if (lane == 0) cst(sr + i, t);
    }
    complete_before();
}

template <int DT, bool VEC>
__device__ inline void draw(const Params& P, uint32_t g, const SeqInfo& in, int lane) {
    const int32_t nsub = P.nsub;
    double* sr = P.sub_r + static_cast<int64_t>(g) * nsub;
    const double u = philox_uniform(P.seed, static_cast<uint32_t>(g + P.b_offset), static_cast<uint32_t>(in.k), 1u);
    double Z, target, before = 0.0;
    int32_t sel;
    bool from_p = false;  // no residual mass left by rounding: draw from p_k
    if (nsub <= kDrawTiles * kWave) {
        double v[kDrawTiles], incl[kDrawTiles];
#pragma unroll
        for (int t = 0; t < kDrawTiles; ++t) v[t] = t * kWave + lane < nsub ? cld(sr + t * kWave + lane) : 0.0;
        Z = regs_scan(v, incl, lane);
        from_p = !(Z > 0.0);
        if (from_p) {
            p_masses<DT, VEC>(P, g, in, sr, lane);
#pragma unroll
            for (int t = 0; t < kDrawTiles; ++t) v[t] = t * kWave + lane < nsub ? cld(sr + t * kWave + lane) : 0.0;
            target = u * regs_scan(v, incl, lane);
        } else {
            target = u * Z;
        }
        sel = regs_find(v, incl, target, lane, before);
    } else {
        Z = scan_total(sr, nsub, lane);
        from_p = !(Z > 0.0);
        if (from_p) p_masses<DT, VEC>(P, g, in, sr, lane);
        target = u * (from_p ? scan_total(sr, nsub, lane) : Z);
        sel = scan_find(sr, nsub, target, lane, before);
    }
    if (P.dbg_z && lane == 0) P.dbg_z[g] = Z * in.scale_p;
    int32_t* out = P.out_tokens + static_cast<int64_t>(g) * (P.gamma + 1) + in.k;
    if (sel < 0) {  // no mass at all (cannot happen for a usable row); keep the output defined
        if (lane == 0) cst(out, -1);
        return;
    }
    const ResidRow rr = resid_row<DT>(P, in, g);
    const bool has_q = rr.qrow != nullptr && !from_p;
    const int64_t j0 = static_cast<int64_t>(sel) * kSub + 16 * lane;
    float xp[16], xq[16];
    load_sub<DT, VEC>(rr, has_q, j0, P.V, xp, xq);
    double mv[16];
    double local = 0.0;
    int32_t mylast = -1;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        mv[v] = static_cast<double>(resid_t(xp[v], xq[v], has_q, P.c32, rr));
        local += mv[v];
        if (mv[v] > 0.0) mylast = static_cast<int32_t>(j0 + v);
    }
    const double incl = before + wave_scan(local, lane);
    const double prev = lane_before(incl);
    const double excl = lane == 0 ? before : prev;
    const uint64_t hit = __ballot(local > 0.0 && excl <= target && target < incl);
    if (hit) {
        const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        if (lane == l) {
            double run = excl;
            int32_t pick = -1;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                run += mv[v];
                if (pick < 0 && mv[v] > 0.0 && run > target) pick = static_cast<int32_t>(j0 + v);
            }
            cst(out, pick >= 0 ? pick : mylast);
        }
    } else {  // rounding: the last element with mass in the subsegment
        const uint64_t mass = __ballot(mylast >= 0);
        const int l = mass ? 63 - __clzll(static_cast<unsigned long long>(mass)) : 0;
        const int32_t pick = __shfl(mylast, l, kWave);
        if (lane == 0) cst(out, pick);
    }
}

// --------------------------------------------------------------------------
// Group finishers and the residual block
// --------------------------------------------------------------------------
// Waits until every statistics block of group g has counted in; false if the
// bounded wait ran out (then the sticky error word is set).
__device__ inline bool wait_published(const Params& P, uint32_t g) {
    const uint32_t* cnt = P.cnt_s + static_cast<int64_t>(g) * kSyncStride;
    const uint32_t want = static_cast<uint32_t>(P.sb);
    if (cld(cnt) == want) return true;
    const uint64_t t0 = wall_clock64();
    for (;;) {
        __builtin_amdgcn_s_sleep(kSleep);
        if (cld(cnt) == want) return true;
        if (wall_clock64() - t0 > kWaitTicks) {
            cst(P.err, 1u);
            return false;
        }
    }
}

// T == 0: the group's last statistics block folds the argmax partials of the
// gamma+1 target rows and runs the greedy accept step (one wavefront).
__device__ inline void finish_greedy(const Params& P, uint32_t g, int lane, char* dyn) {
    __shared__ RowStat rsg[SPEC_MAX_GAMMA + 1];
    const int32_t x = lane < P.gamma ? P.tokens[static_cast<int64_t>(g) * P.gamma + lane] : 0;
    merge_group<true, kWave>(P, g, dyn, rsg);
    (void)accept_wave<true>(P, g, rsg, x, 0.0f, 0.0f, true);
}

// Row statistics: the row's last statistics block folds its partials (one wavefront).
__device__ inline void finish_rows(const Params& P, uint32_t g, int lane) {
    const RowStat o = fold_row_wave(P, static_cast<int64_t>(g) * P.maxp, lane);
    if (lane == 0) {
        P.rows_max[g] = o.m;
        P.rows_sumexp[g] = usable(o.m, o.s) ? o.s : NAN;
    }
}

// T > 0: one residual block of group g (idx in [0, rb)). Once every
// statistics block of g has counted in, the block folds g's partials and
// repeats the accept step (block 0 writes the results); then wavefront w takes
// subsegments idx*4 + w + t*rb*4, t < subs_per_wave(), loading all of them
// before summing. The group's last residual block draws the token and resets
// the group's counters for the next call.
template <int DT, bool VEC>
__device__ inline void resid_block(const Params& P, uint32_t g, uint32_t idx, char* dyn) {
    __shared__ RowStat rs[2 * SPEC_MAX_GAMMA + 1];
    __shared__ SeqInfo shi;
    __shared__ int s_ok;
    __shared__ uint32_t s_last;
    const int lane = static_cast<int>(threadIdx.x & (kWave - 1));
    const int w = static_cast<int>(threadIdx.x / kWave);
    const int32_t gamma = P.gamma;
    // the draft tokens and their two logits do not depend on the statistics:
    // they are loaded before the wait
    int32_t x = 0;
    float lt = 0.0f, ld = 0.0f;
    if (w == 0 && lane < gamma) {
        x = P.tokens[static_cast<int64_t>(g) * gamma + lane];
        if (x >= 0 && x < P.V) {
            lt = load_one<DT>(group_row<DT, kSample>(P, g, static_cast<uint32_t>(lane)), x);
            ld = load_one<DT>(group_row<DT, kSample>(P, g, static_cast<uint32_t>(gamma + 1 + lane)), x);
        }
    }
    if (threadIdx.x == 0) s_ok = wait_published(P, g) ? 1 : 0;
    __syncthreads();
    after_complete();
    SeqInfo in;
    in.k = -1;
    if (s_ok) {
        merge_group<false, kBlock>(P, g, dyn, rs);
        if (w == 0) {
            const SeqInfo si = accept_wave<false>(P, g, rs, x, lt, ld, idx == 0);
            if (lane == 0) shi = si;
        }
        __syncthreads();
        in = shi;
    } else if (idx == 0 && w == 0) {
        // the wait ran out (not expected): the sequence is reported invalid
        if (lane <= gamma) cst(P.out_tokens + static_cast<int64_t>(g) * (gamma + 1) + lane, -1);
        if (lane == 0) cst(P.out_n + g, -1);
    }
    if (in.k >= 0) {
        constexpr int NS = subs_per_wave<DT, VEC>();
        const float c32 = P.c32;
        const ResidRow rr = resid_row<DT>(P, in, g);
        const bool has_q = rr.qrow != nullptr;
        const int32_t stride = P.rb * kWavesPerBlock;
        const int32_t i0 = static_cast<int32_t>(idx) * kWavesPerBlock + w;
        // a lane's 16 elements summed in fp64, in element order (the draw
        // recomputes one subsegment the same way)
        auto lane_sums = [&](const float* xp, const float* xq, int n, double& tr) {
            for (int v = 0; v < n; ++v) tr += static_cast<double>(resid_t(xp[v], xq[v], has_q, c32, rr));
        };
        auto flush = [&](int32_t i, double tr) {
            tr = wave_sum(tr);
            if (lane == 0) cst(P.sub_r + static_cast<int64_t>(g) * P.nsub + i, tr);
        };
        if constexpr (VEC) {
            using SR = SubRaw<DT>;
            SR raw[NS];
#pragma unroll
            for (int t = 0; t < NS; ++t) {
                const int32_t i = i0 + t * stride;
                if (i < P.nsub) raw[t].load(rr, has_q, static_cast<int64_t>(i) * kSub + 16 * lane, P.V);
            }
#pragma unroll
            for (int t = 0; t < NS; ++t) {
                const int32_t i = i0 + t * stride;
                if (i >= P.nsub) break;
                double tr = 0.0;
#pragma unroll
                for (int u = 0; u < SR::NV; ++u) {
                    float xp[SR::EPL], xq[SR::EPL];
                    Chunk<DT, true>::expand(raw[t].p[u], xp);
                    Chunk<DT, true>::expand(raw[t].q[u], xq);
                    lane_sums(xp, xq, SR::EPL, tr);
                }
                flush(i, tr);
            }
        } else {
            for (int32_t i = i0; i < P.nsub; i += stride) {
                float xp[16], xq[16];
                load_sub<DT, false>(rr, has_q, static_cast<int64_t>(i) * kSub + 16 * lane, P.V, xp, xq);
                double tr = 0.0;
                lane_sums(xp, xq, 16, tr);
                flush(i, tr);
            }
        }
    }
    // block arrival: every wavefront's stores have completed before thread 0 counts the block in
    complete_before();
    __syncthreads();
    uint32_t* cnt_r = P.cnt_r + static_cast<int64_t>(g) * kSyncStride;
    if (threadIdx.x == 0)
        s_last = __hip_atomic_fetch_add(cnt_r, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u ==
                 static_cast<uint32_t>(P.rb);
    __syncthreads();
    if (!s_last || w != 0) return;
    after_complete();
    if (lane == 0) {  // every statistics and residual block of g has counted in
        cst(P.cnt_s + static_cast<int64_t>(g) * kSyncStride, 0u);
        cst(cnt_r, 0u);
    }
    if (in.k >= 0) draw<DT, VEC>(P, g, in, lane);
}

// --------------------------------------------------------------------------
// The kernel: one launch per call.
// --------------------------------------------------------------------------
template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kBlock) void k_verify(Params P) {
    extern __shared__ __align__(16) char dyn[];
    int kind;
    uint32_t g, idx;
    decode_block(P, blockIdx.x, kind, g, idx);
    const int lane = static_cast<int>(threadIdx.x & (kWave - 1));
    if (kind == kStatsBlock) {
        __shared__ BlockPieces bp;
        const int w = static_cast<int>(__builtin_amdgcn_readfirstlane(threadIdx.x / kWave));
        const int nwb = min(kWavesPerBlock, P.nw - static_cast<int>(idx) * kWavesPerBlock);  // wavefronts with work
        if (threadIdx.x == 0) bp.done = 0u;
        __syncthreads();
        if (w >= nwb) return;
        const int n = stats_wave<DT, VEC, MODE>(P, g, idx * kWavesPerBlock + w, lane, bp.p[w]);
        // count this wavefront in at the block; the last one writes the block's pieces
        if (lane == 0) bp.n[w] = n;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        uint32_t old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(&bp.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        old = __shfl(old, 0, kWave);
        if (old + 1u != static_cast<uint32_t>(nwb)) return;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        write_pieces<MODE>(P, bp, nwb, lane);
        uint32_t* cnt = P.cnt_s + static_cast<int64_t>(g) * kSyncStride;
        if constexpr (MODE == kSample) {
            // the residual blocks of g watch this count reach sb
            complete_before();
            if (lane == 0) (void)__hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            if (!arrive_last(cnt, static_cast<uint32_t>(P.sb), lane)) return;
            if constexpr (MODE == kGreedy) finish_greedy(P, g, lane, dyn);
            else finish_rows(P, g, lane);
        }
    } else {
        if constexpr (MODE == kSample) resid_block<DT, VEC>(P, g, idx, dyn);
    }
}

// ==========================================================================
// Host side
// ==========================================================================
thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

// Library-owned device memory of one (device, stream). `data` holds the
// partial slots and residual masses, laid out per call shape. `sync` holds the
// group counters at fixed addresses (capacity `groups`): it is cleared when
// allocated and every call leaves its counters at zero again, so calls of any
// shape can follow one another on it.
struct Workspace {
    void* data = nullptr;
    size_t bytes = 0;
    uint32_t* sync = nullptr;
    int64_t groups = 0;
};

std::mutex g_mu;
std::map<std::pair<int, void*>, Workspace> g_ws;  // (device, stream) -> buffers
std::map<int, int> g_cus;                         // device -> compute units

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Layout {
    Params p;  // geometry filled; pointers added at launch
    size_t off_pm, off_pr, off_ps, off_pi, off_subr, bytes;
    int64_t blocks;
    uint32_t lds;
};

int elem_bytes(int32_t dtype) { return dtype == SPEC_F32 ? 4 : 2; }

// Chunk geometry: vector chunks are 1 KiB; scalar chunks are 64 x 4 elements.
int32_t chunk_elems(int32_t dtype, bool vec) { return vec ? kWave * (16 / elem_bytes(dtype)) : kWave * 4; }

// Statistics wavefronts take about kChunksPerWave chunks (many more wavefronts
// than the chip holds at once, which keeps its tail short), but the whole
// problem gets at least 16 wavefronts per compute unit so that small problems
// still spread over the chip. Residual wavefronts take subs_per_wave()
// subsegments of row k each.
Layout plan(int mode, int64_t G, int32_t gamma, int32_t V, int32_t dtype, bool vec, int cus) {
    Layout L{};
    Params& p = L.p;
    const int32_t rps = mode == kSample ? 2 * gamma + 1 : (mode == kGreedy ? gamma + 1 : 1);
    p.G = static_cast<int32_t>(G);
    p.rps = rps;
    p.gamma = gamma;
    p.V = V;
    const int32_t CH = chunk_elems(dtype, vec);
    p.nchunk = (V + CH - 1) / CH;
    const int64_t per_group = static_cast<int64_t>(rps) * p.nchunk;
    const int64_t total = G * per_group;
    const int64_t min_waves = static_cast<int64_t>(cus) * 16;
    int64_t cpw = kChunksPerWave;
    if ((total + cpw - 1) / cpw < min_waves) cpw = (total + min_waves - 1) / min_waves;
    if (cpw > static_cast<int64_t>(kMaxPieces - 1) * p.nchunk) cpw = static_cast<int64_t>(kMaxPieces - 1) * p.nchunk;
    if (cpw < 1) cpw = 1;
    p.cpw = static_cast<int32_t>(cpw);
    p.nw = static_cast<int32_t>((per_group + cpw - 1) / cpw);
    p.sb = (p.nw + kWavesPerBlock - 1) / kWavesPerBlock;
    p.maxp = static_cast<int32_t>((p.nchunk + cpw - 1) / cpw + 1);
    p.nsub = static_cast<int32_t>((static_cast<int64_t>(V) + kSub - 1) / kSub);
    const int spw = vec ? (dtype == SPEC_BF16 ? subs_per_wave<SPEC_BF16, true>() : subs_per_wave<SPEC_F32, true>())
                        : subs_per_wave<SPEC_F32, false>();
    p.rb = mode == kSample ? (p.nsub + kWavesPerBlock * spw - 1) / (kWavesPerBlock * spw) : 0;
    p.lag = p.rb > 0 ? static_cast<int32_t>(G < kLag ? G : kLag) : 0;
    const int64_t gslots = static_cast<int64_t>(rps) * p.maxp;
    p.stage = mode != kRows && gslots <= kMaxStage ? static_cast<int32_t>(gslots) : 0;
    L.blocks = G * (p.sb + p.rb);
    L.lds = static_cast<uint32_t>(p.stage) * 20u;
    const size_t slots = static_cast<size_t>(G) * gslots;
    const size_t subs = mode == kSample ? static_cast<size_t>(G) * p.nsub : 0;
    size_t o = 0;
    L.off_pm = o; o = align_up(o + slots * sizeof(float), 256);
    L.off_pr = o; o = align_up(o + (mode == kGreedy ? 0 : slots) * sizeof(float), 256);
    L.off_ps = o; o = align_up(o + (mode == kGreedy ? 0 : slots) * sizeof(double), 256);
    L.off_pi = o; o = align_up(o + (mode == kGreedy ? slots : 0) * sizeof(int32_t), 256);
    L.off_subr = o; o = align_up(o + subs * sizeof(double), 256);
    L.bytes = o;
    return L;
}

int compute_units(int dev) {
    auto it = g_cus.find(dev);
    if (it != g_cus.end()) return it->second;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 1;
    g_cus[dev] = n;
    return n;
}

// Caller holds g_mu. Grows the buffers of (dev, stream) to `bytes` of data and
// `groups` groups of counters; a new sync buffer is cleared on the stream.
int get_workspace(int dev, hipStream_t stream, size_t bytes, int64_t groups, Workspace** out) {
    Workspace& ws = g_ws[std::make_pair(dev, static_cast<void*>(stream))];
    if (ws.bytes < bytes || ws.groups < groups) {
        if (ws.data || ws.sync)
            if (hipStreamSynchronize(stream) != hipSuccess) return fail(SPEC_EHIP, "hipStreamSynchronize failed");
    }
    if (ws.bytes < bytes) {
        if (ws.data) (void)hipFree(ws.data);
        ws.data = nullptr;
        ws.bytes = 0;
        const size_t want = align_up(bytes + bytes / 4, 1 << 20);
        if (hipMalloc(&ws.data, want) != hipSuccess) {
            ws.data = nullptr;
            (void)hipGetLastError();
            return fail(SPEC_ENOMEM, "hipMalloc of the workspace failed");
        }
        ws.bytes = want;
    }
    if (ws.groups < groups) {
        if (ws.sync) (void)hipFree(ws.sync);
        ws.sync = nullptr;
        ws.groups = 0;
        const int64_t want = static_cast<int64_t>(align_up(static_cast<size_t>(groups + groups / 4), 1024));
        const size_t sbytes = (2 * static_cast<size_t>(want) * kSyncStride + 64) * sizeof(uint32_t);
        if (hipMalloc(reinterpret_cast<void**>(&ws.sync), sbytes) != hipSuccess) {
            ws.sync = nullptr;
            (void)hipGetLastError();
            return fail(SPEC_ENOMEM, "hipMalloc of the workspace failed");
        }
        if (hipMemsetAsync(ws.sync, 0, sbytes, stream) != hipSuccess) {
            (void)hipFree(ws.sync);
            ws.sync = nullptr;
            return fail(SPEC_EHIP, "hipMemsetAsync of the workspace failed");
        }
        ws.groups = want;
    }
    *out = &ws;
    return SPEC_OK;
}

void bind_workspace(Layout& L, Workspace& ws) {
    char* base = static_cast<char*>(ws.data);
    Params& p = L.p;
    p.part_m = reinterpret_cast<float*>(base + L.off_pm);
    p.part_r = reinterpret_cast<float*>(base + L.off_pr);
    p.part_s = reinterpret_cast<double*>(base + L.off_ps);
    p.part_i = reinterpret_cast<int32_t*>(base + L.off_pi);
    p.sub_r = reinterpret_cast<double*>(base + L.off_subr);
    const int64_t words = ws.groups * kSyncStride;
    p.cnt_s = ws.sync;
    p.cnt_r = ws.sync + words;
    p.err = ws.sync + 2 * words;
}

// Timing events, when given, are bound to the kernel dispatch itself (its
// start and end timestamps), so they add no packets to the stream.
template <int DT, bool VEC>
void launch_t(int mode, const Layout& L, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    const dim3 grid(static_cast<unsigned>(L.blocks)), block(kBlock);
    if (mode == kSample)
        hipExtLaunchKernelGGL((k_verify<DT, VEC, kSample>), grid, block, L.lds, st, e0, e1, 0, L.p);
    else if (mode == kGreedy)
        hipExtLaunchKernelGGL((k_verify<DT, VEC, kGreedy>), grid, block, L.lds, st, e0, e1, 0, L.p);
    else
        hipExtLaunchKernelGGL((k_verify<DT, VEC, kRows>), grid, block, L.lds, st, e0, e1, 0, L.p);
}

void launch(int32_t dtype, bool vec, int mode, const Layout& L, hipStream_t st, hipEvent_t e0 = nullptr,
            hipEvent_t e1 = nullptr) {
    if (dtype == SPEC_F32) {
        if (vec) launch_t<SPEC_F32, true>(mode, L, st, e0, e1);
        else launch_t<SPEC_F32, false>(mode, L, st, e0, e1);
    } else {
        if (vec) launch_t<SPEC_BF16, true>(mode, L, st, e0, e1);
        else launch_t<SPEC_BF16, false>(mode, L, st, e0, e1);
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

float fold_temperature(float T) { return static_cast<float>(1.4426950408889634 / static_cast<double>(T)); }

int check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SPEC_EHIP, std::string(what) + ": " + hipGetErrorString(e));
    return SPEC_OK;
}

// Size limits: chunk counts are 32-bit on the device, and a dispatch holds
// fewer than 2^32 work-items.
int check_size(const Layout& L) {
    const int64_t chunks = static_cast<int64_t>(L.p.G) * L.p.rps * L.p.nchunk;
    if (chunks >= (int64_t(1) << 31) || L.blocks * kBlock >= (int64_t(1) << 32) || L.blocks < 1)
        return fail(SPEC_EINVAL, "problem too large");
    return SPEC_OK;
}

}  // namespace

// ==========================================================================
// C ABI
// ==========================================================================
extern "C" {

int32_t spec_verify_abi_version(void) { return 1; }

const char* spec_verify_last_error(void) { return g_last_error.c_str(); }

size_t spec_verify_workspace_bytes(int32_t B, int32_t gamma, int32_t V, int32_t dtype, float temperature) {
    if (B < 1 || gamma < 1 || gamma > SPEC_MAX_GAMMA || V < 1 || (dtype != SPEC_F32 && dtype != SPEC_BF16))
        return 0;
    int dev = 0;
    (void)hipGetDevice(&dev);
    const bool vec = (static_cast<int64_t>(V) * elem_bytes(dtype)) % 16 == 0;
    std::lock_guard<std::mutex> lk(g_mu);
    const Layout L = plan(temperature == 0.0f ? kGreedy : kSample, B, gamma, V, dtype, vec, compute_units(dev));
    return L.bytes + (2 * static_cast<size_t>(B) * kSyncStride + 64) * sizeof(uint32_t);
}

void spec_verify_release_workspace(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto& kv : g_ws) {
        if (!kv.second.data && !kv.second.sync) continue;
        (void)hipSetDevice(kv.first.first);
        (void)hipStreamSynchronize(static_cast<hipStream_t>(kv.first.second));
        if (kv.second.data) (void)hipFree(kv.second.data);
        if (kv.second.sync) (void)hipFree(kv.second.sync);
    }
    g_ws.clear();
    (void)hipSetDevice(cur);
}

int spec_verify_ex(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                   int32_t B, int32_t gamma, int32_t V, int32_t dtype, float temperature, uint64_t seed,
                   int32_t* out_tokens, int32_t* out_n_accepted, void* stream,
                   const spec_extras_t* extras) {
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return fail(SPEC_EDTYPE, "dtype must be SPEC_F32 or SPEC_BF16");
    if (B < 1) return fail(SPEC_EINVAL, "B must be >= 1");
    if (gamma < 1 || gamma > SPEC_MAX_GAMMA) return fail(SPEC_EINVAL, "gamma must be in [1, 63]");
    if (V < 1) return fail(SPEC_EINVAL, "V must be >= 1");
    if (!(temperature >= 0.0f)) return fail(SPEC_EINVAL, "temperature must be >= 0 and not NaN");
    const bool greedy = temperature == 0.0f;
    if (!target_logits || !draft_tokens || !out_tokens || !out_n_accepted)
        return fail(SPEC_EINVAL, "null pointer argument");
    if (!greedy && !draft_logits) return fail(SPEC_EINVAL, "draft_logits may be NULL only at temperature 0");
    const float c32 = greedy ? 0.0f : fold_temperature(temperature);
    if (!greedy && !(std::isfinite(c32) && c32 > 0.0f))
        return fail(SPEC_EINVAL, "temperature too small or too large for fp32 exponent scaling");
    const bool vec = (static_cast<int64_t>(V) * elem_bytes(dtype)) % 16 == 0 && aligned16(target_logits) &&
                     (greedy || aligned16(draft_logits));
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPEC_EHIP, "hipGetDevice failed");
    const int mode = greedy ? kGreedy : kSample;

    std::lock_guard<std::mutex> lk(g_mu);
    Layout L = plan(mode, B, gamma, V, dtype, vec, compute_units(dev));
    if (int rc = check_size(L)) return rc;
    Workspace* ws = nullptr;
    if (int rc = get_workspace(dev, st, L.bytes, L.p.G, &ws)) return rc;
    bind_workspace(L, *ws);
    Params& p = L.p;
    p.c32 = c32;
    p.seed = seed;
    p.b_offset = extras ? extras->b_offset : 0;
    p.tgt = target_logits;
    p.dft = greedy ? nullptr : draft_logits;
    p.tokens = draft_tokens;
    p.out_tokens = out_tokens;
    p.out_n = out_n_accepted;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (extras) {
        p.dbg_row_max = extras->row_max;
        p.dbg_row_sumexp = extras->row_sumexp;
        p.dbg_p = extras->p_draft;
        p.dbg_q = extras->q_draft;
        p.dbg_z = extras->Z;
        p.dbg_argmax = extras->argmax;
        e0 = static_cast<hipEvent_t>(extras->events[0]);
        e1 = static_cast<hipEvent_t>(extras->events[1]);
    }
    launch(dtype, vec, mode, L, st, e0, e1);
    return check_launch("verification kernel");
}

int spec_verify(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                int32_t B, int32_t gamma, int32_t V, int32_t dtype, float temperature, uint64_t seed,
                int32_t* out_tokens, int32_t* out_n_accepted, void* stream) {
    return spec_verify_ex(target_logits, draft_logits, draft_tokens, B, gamma, V, dtype, temperature, seed,
                          out_tokens, out_n_accepted, stream, nullptr);
}

int spec_row_stats(const void* logits, int64_t rows, int32_t V, int32_t dtype, float temperature,
                   float* row_max, double* row_sumexp, void* stream) {
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return fail(SPEC_EDTYPE, "dtype must be SPEC_F32 or SPEC_BF16");
    if (rows < 1 || V < 1) return fail(SPEC_EINVAL, "rows and V must be >= 1");
    if (rows >= (int64_t(1) << 31)) return fail(SPEC_EINVAL, "problem too large");
    if (!(temperature > 0.0f)) return fail(SPEC_EINVAL, "temperature must be > 0");
    if (!logits || !row_max || !row_sumexp) return fail(SPEC_EINVAL, "null pointer argument");
    const float c32 = fold_temperature(temperature);
    if (!(std::isfinite(c32) && c32 > 0.0f)) return fail(SPEC_EINVAL, "temperature out of range");
    const bool vec = (static_cast<int64_t>(V) * elem_bytes(dtype)) % 16 == 0 && aligned16(logits);
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPEC_EHIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(g_mu);
    Layout L = plan(kRows, rows, 1, V, dtype, vec, compute_units(dev));
    if (int rc = check_size(L)) return rc;
    Workspace* ws = nullptr;
    if (int rc = get_workspace(dev, st, L.bytes, L.p.G, &ws)) return rc;
    bind_workspace(L, *ws);
    L.p.c32 = c32;
    L.p.tgt = logits;
    L.p.rows_max = row_max;
    L.p.rows_sumexp = row_sumexp;
    launch(dtype, vec, kRows, L, st);
    return check_launch("statistics kernel");
}

}  // extern "C"
