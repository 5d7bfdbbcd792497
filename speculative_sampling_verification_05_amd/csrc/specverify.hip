// specverify.hip - batched speculative-sampling verification for gfx950.
//
// Pages (cited by title and section):
//  [Ch15] "Chapter 15: Decoding acceleration techniques" (zsc.github.io, LLM
//         edge inference), 15.1.2: step 2 (softmax of every verified row),
//         step 3 (accept with probability min(1, p/q), stop at the first
//         rejection: the early stop), step 4 (resample from max(0, p - q)/Z);
//         15.1.4 (the probability gather); 15.4.2 (fused kernels, low-precision
//         inputs with fp32 accumulation, coalesced loads).
//  [CSDN] devpress.csdn.net speculative-inference post, 2.1: the
//         speculative_decode() loop (strict u < alpha, residual clamp).
//  [HSD]  "LLM inference optimisation: hidden-state speculative decoding", 3.3:
//         the bonus token drawn from the last target row.
//
// One kernel launch per call. Its grid is laid out position by position: a
// unit is one (position i, sequence b) - at T > 0 the pair (target row i,
// draft row i) for i < gamma and the bonus row gamma alone, at T == 0 target
// row i, for the stand-alone row statistics one row - and the units of
// position 0 come first, then position 1, and so on.
//  statistics blocks  stream a unit's rows once. Each wavefront owns a
//                     contiguous range of 1 KiB chunks of the unit's rows,
//                     keeps per lane an online max and a sum of 2^(x*c - R)
//                     (R an integer reference, c = log2(e)/T), software-
//                     pipelines its 16-byte non-temporal loads and writes one
//                     partial per row piece; at T == 0 it tracks the first
//                     index of the maximum instead. The unit's last block to
//                     count in folds the partials and takes the accept step of
//                     position i (alpha in fp64 from the draft token's two
//                     logits, the Philox uniform), then reads the decision
//                     words of the sequence's earlier positions: if they were
//                     all accepted it publishes its own, and if position i ends
//                     the sequence (a rejection, an unusable row, or the bonus
//                     row after gamma acceptances) it writes the outputs and
//                     the sequence's draw record.
//  early stop         a wavefront whose sequence is already known to have
//                     stopped at an earlier position loads nothing, so rows
//                     after a sequence's first rejection are mostly never read.
//  residual blocks    (T > 0) close the grid, one set per sequence. Once the
//                     sequence's draw record is out they load the stopping
//                     row's target and draft columns into registers, sum the
//                     residual max(0, p - q) (or p for the bonus row) in fp64,
//                     exchange block sums, and the block, wavefront, lane and
//                     element where the cumulative mass crosses u*Z are found
//                     in ascending index order from the registers.
// A block waits only for blocks of lower index (earlier positions, or its own
// sequence's residual blocks, which follow one another), which the in-order
// dispatch has already started, and every wait is bounded in time. Data
// crossing blocks moves through device-coherent (agent-scope) atomic loads and
// stores, which bypass the per-XCD L2 caches, ordered by waiting for their
// completion; decision words and draw records carry the call's epoch, so
// nothing of them has to be cleared between calls.
// Exponentials are fp32 (v_exp_f32 on one FMA); every sum and comparison that
// decides a token is fp64.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
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
#define SPECVERIFY_CHUNKS_PER_WAVE 32
#endif
#ifndef SPECVERIFY_GREEDY_CHUNKS_PER_WAVE
#define SPECVERIFY_GREEDY_CHUNKS_PER_WAVE 8
#endif
#ifndef SPECVERIFY_GREEDY_CHUNKS_PER_WAVE_BF16
#define SPECVERIFY_GREEDY_CHUNKS_PER_WAVE_BF16 12
#endif
#ifndef SPECVERIFY_GROUP_CHUNKS_PER_WAVE
#define SPECVERIFY_GROUP_CHUNKS_PER_WAVE 24
#endif
#ifndef SPECVERIFY_LAG
#define SPECVERIFY_LAG 56
#endif
#ifndef SPECVERIFY_BF16_SUBS
#define SPECVERIFY_BF16_SUBS 2
#endif
#ifndef SPECVERIFY_SLEEP
#define SPECVERIFY_SLEEP 2
#endif
#ifndef SPECVERIFY_DRAFT_CW
#define SPECVERIFY_DRAFT_CW 4
#endif
#ifndef SPECVERIFY_CACHED_TAIL_MB
#define SPECVERIFY_CACHED_TAIL_MB 128
#endif
#ifndef SPECVERIFY_NEAR_COUNT
#define SPECVERIFY_NEAR_COUNT 4
#endif
#ifndef SPECVERIFY_SYNC_STRIDE
#define SPECVERIFY_SYNC_STRIDE 64
#endif

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kUnroll = SPECVERIFY_STATS_UNROLL;           // chunks per pipelined load group
constexpr int kChunksPerWave = SPECVERIFY_CHUNKS_PER_WAVE;  // 1 KiB chunks per statistics wavefront (position-major)
// (position-major at T == 0: short ranges put each position's decision out
// sooner, so the early stop skips more rows. Measured on the greedy recipe
// (fp32, V = 128256), 8 against 16 chunks: 24.0 against 28.5 us at 32
// sequences, 42.5 against 49.9 at 64, 68.8 against 75.4 at 128, 117.8
// against 125.7 at 256, 15.9 against 16.7 at 16 (4, 6, 10 and 12 chunks in
// between or worse). bf16 rows, 12 against 8 and 16 chunks: 47.5 against 53.6
// and 48.9 us at 256 sequences of V = 152064, 29.4 against 30.4 and 30.2 at
// 128 of V = 128256, 17.6 against 16.6 and 18.8 at 32)
constexpr int kGreedyChunksPerWave = SPECVERIFY_GREEDY_CHUNKS_PER_WAVE;
constexpr int kGreedyChunksPerWaveBf16 = SPECVERIFY_GREEDY_CHUNKS_PER_WAVE_BF16;
constexpr int kGroupChunksPerWave = SPECVERIFY_GROUP_CHUNKS_PER_WAVE;  // (group-major)
// group-major: groups between a group's statistics blocks and its residual
// blocks. Past that many groups the first groups' closing steps start before
// the stream ends. Measured on the headline recipe against all residual
// blocks at the end: 53.7 against 54.1 us at 64 sequences, 76.5 against 78.7
// at 96 (lags 40 and 48: 55.8 and 54.3 at 64, 77.7 and 76.2 at 96).
constexpr int kLag = SPECVERIFY_LAG;
// group-major in two phases: groups between a group's first-phase statistics
// blocks and its decider, once there are more than twice as many groups (else
// all deciders follow the first phase). Measured on the headline recipe
// against all deciders after the first phase: 72.3 against 78.6 us at
// B = 128, 104.5 against 109.2 at 192, 61.4 against 62.9 at 96, but 50.8
// against 50.3 at 64 (lags 8, 16, 24 within 0.5 us of 32).
#ifndef SPECVERIFY_DECIDE_LAG
#define SPECVERIFY_DECIDE_LAG 32
#endif
constexpr int kDecideLag = SPECVERIFY_DECIDE_LAG;
// Two phases: chunks per second-phase wavefront from this many groups on
// (below it the first phase's). Measured on the headline recipe, 48 against
// 24: 70.9 against 72.2 us at B = 128, 101.6 against 104.5 at 192, but 58.9
// against 58.2 at 96 and 50.5 against 46.2 at 64 (32 and 64 chunks: 47.7
// and 51.8 at 64, 72.3 and 72.1 at 128).
constexpr int64_t kLongPhase2Groups = 128;
constexpr int64_t kPhase2ChunksPerWave = 48;
// Two phases: a second-phase statistics block waits for its group's record
// before it loads (1), or reads it once and loads unless it already says stop (0).
#ifndef SPECVERIFY_PHASE2_WAIT
#define SPECVERIFY_PHASE2_WAIT 1
#endif
// group-major, T > 0: the last groups, about this many bytes of rows, are
// streamed with ordinary loads (the rest non-temporal), so that the closing
// steps, which follow the end of the stream, re-read row k from the caches
constexpr int64_t kCachedTailBytes = static_cast<int64_t>(SPECVERIFY_CACHED_TAIL_MB) << 20;
constexpr int kSub = kWave * 16;            // group-major: elements per residual subsegment
constexpr int kMaxStage = 1024;             // group-major: partial slots of one group staged in LDS
constexpr int kHold = 8;                    // chunks a draw wavefront holds in registers
constexpr int kPairCw = kHold / 2;          // of each row: target and draft
constexpr float kRUnset = -1.0e30f;         // reference before the first finite value
constexpr uint64_t kWaitTicks = 200000000ull;        // default bound on a wait, and the drain bound: 2 s at 100 MHz
constexpr int kSleep = SPECVERIFY_SLEEP;             // s_sleep argument between polls (64 cycles each)
constexpr int kSyncStride = SPECVERIFY_SYNC_STRIDE;  // words between two counters
constexpr int kRecWords = 32;               // per sequence: draw record (tag + 3 data words), then its two
                                            // ticket counters, each on a 128-byte line of its own
constexpr int kClaimWord = 16;              // tickets handed out for the draw's pieces
constexpr int kPieceWord = 24;              // pieces counted in

enum : int { kSample = 0, kGreedy = 1, kRows = 2 };
enum : int { kStatsBlock = 0, kResidBlock = 1, kDecideBlock = 2 };
// decision word status (low bits; the high 32 bits hold the call's epoch)
enum : uint32_t { kPending = 0, kAcc = 1, kRej = 2, kBad = 3 };
// what the decision words of positions < i say about a sequence
enum : int { kLive = 0, kStopped = 1, kUnknown = 2, kTimedOut = 3 };
// draw record kinds
enum : uint32_t { kNoDraw = 0, kDrawResidual = 1, kDrawP = 2 };

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

// Logits read once go straight into registers: 16-byte non-temporal loads.
// Rows read twice in close succession (the expected-acceptance launch) use
// ordinary loads (NT false), so that the second read finds them in the cache.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <bool NT = true>
__device__ inline uint4 load_stream(const char* p) {
    u32x4 v;
    if constexpr (NT) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else v = *reinterpret_cast<const u32x4*>(p);
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

    template <bool NT = true>
    __device__ static inline Raw load_full(const char* row, int64_t c, int lane) {
        if constexpr (VEC) {
            return load_stream<NT>(row + (c * CH + lane * EPL) * ElemBytes<DT>::value);
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
    template <bool NT = true>
    __device__ static inline Raw load_clamped(const char* row, int64_t c, int64_t c_last, int lane, int32_t V) {
        const int64_t cc = c <= c_last ? c : c_last;
        if constexpr (VEC) {
            const int64_t e = cc * CH + lane * EPL;
            return load_stream<NT>(row + (e < V ? e : cc * CH) * ElemBytes<DT>::value);  // V % EPL == 0 here
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
    // A chunk past the end of the row: -inf everywhere (no mass, never a maximum).
    __device__ static inline Raw blank() {
        if constexpr (VEC) {
            const uint32_t ninf = DT == SPEC_F32 ? 0xFF800000u : 0xFF80FF80u;
            return make_uint4(ninf, ninf, ninf, ninf);
        } else {
            return make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
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
// The value of lane l - 1 (0 in lane 0).
__device__ inline double lane_before(double v) { return dpp_f64<0x138, 0xF>(v); }

// --------------------------------------------------------------------------
// Device-coherent access. Agent-scope atomic loads and stores bypass the L2
// cache of the XCD that issues them, so what one block publishes is read
// unchanged by a block on another XCD.
// --------------------------------------------------------------------------
__device__ inline float cld(const float* p) {
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
}
__device__ inline int32_t cld(const int32_t* p) {
    return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
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
__device__ inline double cld(const double* p) {
    return __longlong_as_double(static_cast<long long>(
        __hip_atomic_load(reinterpret_cast<unsigned long long*>(const_cast<double*>(p)), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT)));
}

__device__ inline void cst64(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t cld64(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
// Bounded spin: polls pred() (wave-uniform, or called by a single lane), with
// a short sleep between polls, until it holds (true) or more than `ticks` of
// the device's constant-rate wall clock have passed since the first failed
// poll (false). Every wait below waits only for blocks of lower index, which
// in-order dispatch has already started, so in correct operation it ends; the
// bound is the failure detector. A wait that gives up sets the sticky error
// word, reports what it owns as invalid, and then drains: it goes on waiting,
// up to kWaitTicks, for the same condition, so that the counters it would
// reset are left at zero for the next call.
template <class Pred>
__device__ inline bool spin_until(Pred pred, uint64_t ticks) {
    if (pred()) return true;
    const uint64_t t0 = wall_clock64();
    for (;;) {
        __builtin_amdgcn_s_sleep(kSleep);
        if (pred()) return true;
        if (wall_clock64() - t0 > ticks) return false;
    }
}
// The same wait for *cnt == want (one lane). While more than kNearCount
// counts are missing it polls one at a time; then with three polls in flight,
// a poll issued whenever the oldest returns, so that the last count is seen
// about one round trip after it lands rather than up to two (polling that fast
// all along would load the memory system while the stream runs).
__device__ inline bool spin_count(const uint32_t* cnt, uint32_t want, uint64_t ticks) {
    const uint64_t t0 = wall_clock64();
    for (;;) {
        const uint32_t v = cld(cnt);
        if (v == want) return true;
        if (v + SPECVERIFY_NEAR_COUNT >= want) break;
        if (wall_clock64() - t0 > ticks) return false;
        __builtin_amdgcn_s_sleep(kSleep);
    }
    uint32_t a = cld(cnt);
    __builtin_amdgcn_s_sleep(kSleep);
    uint32_t b = cld(cnt);
    __builtin_amdgcn_s_sleep(kSleep);
    uint32_t c = cld(cnt);
    for (;;) {
        if (a == want) return true;
        a = cld(cnt);
        if (b == want) return true;
        b = cld(cnt);
        if (c == want) return true;
        c = cld(cnt);
        if (wall_clock64() - t0 > ticks) return false;
        __builtin_amdgcn_s_sleep(kSleep);
    }
}
// --------------------------------------------------------------------------
// Launch geometry and arguments
// --------------------------------------------------------------------------
struct Params {
    int32_t B;       // sequences (rows for the stand-alone statistics)
    int32_t gamma;
    int32_t V;
    int32_t nchunk;  // chunks per row
    int32_t cpw;     // chunks per statistics wavefront
    int32_t maxp;    // partial slots per row (a row spans at most maxp wavefronts)
    int32_t nw2;     // statistics wavefronts of a two-row unit
    int32_t nb2;     //   and its blocks
    int32_t nw1;     // statistics wavefronts of a one-row unit
    int32_t nb1;     //   and its blocks
    int32_t nbr;     // pieces of a draw, and closing blocks per sequence (T > 0)
    int32_t cstride; // words between two counters
    int32_t rps;     // group-major: rows per group (2*gamma+1)
    int32_t nw;      // group-major: statistics wavefronts per group
    int32_t sb;      //   statistics blocks per group
    int32_t rb;      //   residual blocks per group
    int32_t lag;     //   groups between a group's statistics blocks and its residual blocks
    int32_t nsub;    //   residual subsegments per row
    int32_t stage;   //   a group's partial slots staged in LDS, or 0 (fold from memory)
    int32_t cached_from;  // group-major: groups from here on stream with ordinary loads, which keep
                          //   the rows in the caches for the residual blocks' re-read of row k
    int32_t spw;     // group-major: residual subsegments per wavefront (1, or subs_per_wave())
    int32_t srows;   // group-major: rows of a group the statistics blocks stream (rps, or rps - 1
                     //   when the bonus row is deferred)
    int32_t defer;   // group-major, T > 0: the bonus row is not streamed; the closing blocks of a
                     //   sequence that accepts all gamma tokens read it (no per-row debug output)
    int32_t p0;      // group-major in two phases (0: one phase): the first p0 row pairs of every
    int32_t pnw2;    //   group, then the group's decider, then the other pairs (their wavefronts
    int32_t psb2;    //   and blocks per group), read only for sequences not stopped within p0
    int32_t cpw2;    //   chunks per statistics wavefront in the second phase
    int32_t skip;    // early stop: wavefronts of sequences already stopped load nothing
    uint32_t epoch;  // tag of this call's decision words and draw records (never 0)
    uint64_t wait;   // bound on a wait, in wall-clock ticks (kWaitTicks unless the host set another)
    float c32;       // log2(e)/T
    uint64_t seed;
    int64_t b_offset;
    const void* tgt;
    const void* dft;
    const int32_t* tokens;
    int32_t* out_tokens;
    int32_t* out_n;
    int64_t rows_split;   // row statistics: rows from here on are read from dft (row - rows_split)
    float* rows_max;      // row statistics outputs
    double* rows_sumexp;
    uint32_t* tree_done;  // row statistics of a tree call, or null: per tree (kSyncStride words apart) the
                          //   finished rows, counted after their coherent stores
    int32_t tree_n;       //   nodes per tree (row r < rows_split belongs to tree r / tree_n)
    int32_t tgt_group;    // row statistics: 0, or row r < rows_split is target row
                          //   (r / tgt_group) * (tgt_group + 1) + r % tgt_group (each sequence's bonus row skipped)
    int32_t pair_rows;    // row statistics: 1 if row r is row r % 2 (0 target, 1 draft) of position pair r / 2
                          //   (the target row mapped with tgt_group)
    float* part_m;        // [units][2][maxp] per partial slot: max of the piece
    float* part_r;        //   integer reference of the piece (T > 0)
    double* part_s;       //   sum of 2^(x*c - reference) (T > 0)
    int32_t* part_i;      //   first index of the maximum (T == 0)
    float* tok_l;         // [units][2] the draft token's target and draft logits (T > 0)
    double* msum;         // [B][nbr*4] masses of the draw's wavefronts
    uint32_t* cnt;        // unit counters, `cstride` words apart
    uint64_t* dec;        // [B][gamma+1] decision words: epoch << 32 | status
    uint64_t* rec;        // [B][kRecWords] draw records and their ticket counters
    double* sub_r;        // group-major: [B][nsub] residual mass per subsegment (t units)
    float* sub_R;         // group-major, deferred bonus row: [B][nsub] each subsegment mass's reference
    uint32_t* cnt_s;      // group-major: [B] statistics blocks counted in, kSyncStride words apart
    uint32_t* cnt_r;      // group-major: [B] residual blocks counted in
    uint32_t* err;        // sticky: a wait ran out
    float* dbg_row_max;
    double* dbg_row_sumexp;
    double* dbg_p;
    double* dbg_q;
    double* dbg_z;
    int32_t* dbg_argmax;
};

// A block's role. Statistics units are numbered i*B + b (position-major; the
// row index for the stand-alone statistics) and take nb consecutive blocks:
// nb2 for a target/draft pair (T > 0, i < gamma), nb1 for one row. At T > 0
// the residual blocks of sequence 0, 1, ... follow, nbr each.
struct Role {
    int kind;
    uint32_t unit;  // statistics unit, or sequence of a residual block
    int32_t i;      // position (0..gamma)
    int32_t b;      // sequence, or row
    int32_t r;      // block within the unit (or the sequence's residual blocks)
    int32_t rows;   // rows of the unit (1 or 2)
    int32_t nw;     // wavefronts of the unit
    int32_t nb;     // blocks of the unit
};
template <int MODE>
__device__ inline Role role_at(const Params& P, uint32_t x);
template <int MODE>
__device__ inline Role role_of(const Params& P) { return role_at<MODE>(P, blockIdx.x); }
template <int MODE>
__device__ inline Role role_at(const Params& P, uint32_t x) {
    const uint32_t B = static_cast<uint32_t>(P.B);
    Role o;
    o.kind = kStatsBlock;
    if constexpr (MODE == kRows) {
        const uint32_t nb = static_cast<uint32_t>(P.nb1);
        o.unit = x / nb;
        o.r = static_cast<int32_t>(x - o.unit * nb);
        o.i = 0;
        o.b = static_cast<int32_t>(o.unit);
        o.rows = 1;
        o.nw = P.nw1;
        o.nb = P.nb1;
        return o;
    }
    const uint32_t G = static_cast<uint32_t>(P.gamma);
    if constexpr (MODE == kSample) {
        const uint32_t nb2 = static_cast<uint32_t>(P.nb2), pairs = G * B * nb2;
        if (x < pairs) {
            o.unit = x / nb2;
            o.r = static_cast<int32_t>(x - o.unit * nb2);
            o.i = static_cast<int32_t>(o.unit / B);
            o.b = static_cast<int32_t>(o.unit - static_cast<uint32_t>(o.i) * B);
            o.rows = 2;
            o.nw = P.nw2;
            o.nb = P.nb2;
            return o;
        }
        x -= pairs;
        const uint32_t nb1 = static_cast<uint32_t>(P.nb1), bonus = B * nb1;
        if (x >= bonus) {
            x -= bonus;
            const uint32_t nbr = static_cast<uint32_t>(P.nbr);
            o.kind = kResidBlock;
            o.b = static_cast<int32_t>(x / nbr);
            o.unit = static_cast<uint32_t>(o.b);
            o.r = static_cast<int32_t>(x - static_cast<uint32_t>(o.b) * nbr);
            o.i = 0;
            o.rows = 2;
            o.nw = 0;
            o.nb = P.nbr;
            return o;
        }
        const uint32_t bb = x / nb1;
        o.unit = G * B + bb;
        o.r = static_cast<int32_t>(x - bb * nb1);
        o.i = static_cast<int32_t>(G);
        o.b = static_cast<int32_t>(bb);
        o.rows = 1;
        o.nw = P.nw1;
        o.nb = P.nb1;
        return o;
    } else {  // greedy: every unit is one target row
        const uint32_t nb1 = static_cast<uint32_t>(P.nb1);
        o.unit = x / nb1;
        o.r = static_cast<int32_t>(x - o.unit * nb1);
        o.i = static_cast<int32_t>(o.unit / B);
        o.b = static_cast<int32_t>(o.unit - static_cast<uint32_t>(o.i) * B);
        o.rows = 1;
        o.nw = P.nw1;
        o.nb = P.nb1;
        return o;
    }
}

// Row j of a unit: the target row i, then (two-row units) the draft row i.
template <int DT, int MODE>
__device__ inline const char* unit_row(const Params& P, const Role& U, int32_t j) {
    if constexpr (MODE == kRows) {
        int64_t r = U.b;
        if (P.pair_rows) {
            if (r & 1) return row_at<DT>(P.dft, (r >> 1) * P.V);
            r >>= 1;
        } else if (r >= P.rows_split) {
            return row_at<DT>(P.dft, (r - P.rows_split) * P.V);
        }
        const int64_t g = P.tgt_group;
        return row_at<DT>(P.tgt, (g > 0 ? (r / g) * (g + 1) + r % g : r) * P.V);
    } else {
        if (j == 0) return row_at<DT>(P.tgt, (static_cast<int64_t>(U.b) * (P.gamma + 1) + U.i) * P.V);
        return row_at<DT>(P.dft, (static_cast<int64_t>(U.b) * P.gamma + U.i) * P.V);
    }
}
__device__ inline int64_t slot_base(const Params& P, uint32_t unit, int32_t j) {
    return (static_cast<int64_t>(unit) * 2 + j) * P.maxp;
}

// The statistics blocks at the head of the grid (groups [0, D), S blocks
// each): in chunks of 8 groups, group c*8 + k takes the blocks x with
// x % 8 == k, so that all its blocks run on one XCD (consecutive blocks go
// to the XCDs in turn) and it finishes with that XCD rather than with the
// slowest of the eight; a last chunk of fewer than 8 groups keeps its blocks
// in order. Measured against blocks in group order: 45.3 against 46.2 us on
// the headline recipe, 26.2 against 27.7 at B = 16, 41.9 against 42.5 at
// B = 48, 16.5 against 17.3 on the 8-sequence fp32 workload; unchanged at
// B = 4, 32 and from 96 on.
__device__ inline void head_block(uint32_t x, uint32_t S, uint32_t D, uint32_t& g, uint32_t& idx) {
    const uint32_t full = (D >> 3) * 8u * S;
    if (x < full) {
        const uint32_t c = x / (8u * S), j = x - c * 8u * S;
        g = c * 8u + (j & 7u);
        idx = j >> 3;
        return;
    }
    g = x / S;
    idx = x - g * S;
}

// Group-major grid (a group is one sequence, all 2*gamma+1 rows). Grid order:
// groups [0, lag) contribute their statistics blocks (one XCD per group, as
// head_block places them); each group
// j in [lag, G) then contributes its statistics blocks followed by the
// residual blocks of group j - lag; the residual blocks of the last lag groups
// close the grid. A group's residual blocks thus always follow all of its
// statistics blocks.
// In two phases (p0 > 0) the order is: every group's first-phase statistics
// blocks, one decider per group, every group's second-phase statistics
// blocks, every group's residual blocks; each waits only for earlier blocks.
__device__ inline void decode_block(const Params& P, uint32_t x, int& kind, uint32_t& g, uint32_t& idx, int& phase) {
    const uint32_t S = static_cast<uint32_t>(P.sb), R = static_cast<uint32_t>(P.rb);
    const uint32_t D = static_cast<uint32_t>(P.lag), G = static_cast<uint32_t>(P.B);
    phase = 0;
    if (P.p0 > 0) {
        // (the decider of group g follows the first-phase blocks of group
        // g + D, D = P.lag, so that it decides while the first phase streams)
        const uint32_t S2 = static_cast<uint32_t>(P.psb2);
        const uint32_t head = D * S, mid = (G - D) * (S + 1);
        if (x < head) {
            kind = kStatsBlock;
            phase = 1;
            head_block(x, S, D, g, idx);
        } else if ((x -= head) < mid) {
            const uint32_t t = x / (S + 1), o = x - t * (S + 1);
            if (o < S) {
                kind = kStatsBlock;
                phase = 1;
                g = D + t;
                idx = o;
            } else {
                kind = kDecideBlock;
                g = t;
                idx = 0;
            }
        } else if ((x -= mid) < D) {
            kind = kDecideBlock;
            g = G - D + x;
            idx = 0;
        } else if ((x -= D) < G * S2) {
            kind = kStatsBlock;
            phase = 2;
            g = x / S2;
            idx = x - g * S2;
        } else {
            // (the residual blocks too with one XCD per group: 45.0 against
            // 45.4 us on the headline recipe, 69.9 against 71.0 at B = 128,
            // 100.0 against 102.3 at 192; the second-phase blocks placed so
            // measured 48.7 against 45.4 at the headline)
            x -= G * S2;
            kind = kResidBlock;
            head_block(x, R, G, g, idx);
        }
        return;
    }
    const uint32_t head = D * S;
    if (x < head) {
        kind = kStatsBlock;
        head_block(x, S, D, g, idx);
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
    // (one XCD per group here too measured mixed: 33.8 against 34.4 us at
    // B = 32 and 15.8 against 16.7 on the 8-sequence fp32 workload, but 27.0
    // against 26.8 at B = 16 and 22.1 against 21.7 at B = 4; not kept)
    const uint32_t t = x / R;
    g = (G - D) + t;
    idx = x - t * R;
}

// The group row (target rows 0..gamma, then draft rows) of stream row j of a
// group's statistics blocks. One phase: every row, but with the bonus row
// deferred the rows after target row gamma - 1 are the draft rows. First
// phase (1): target rows 0..p0-1, then draft rows 0..p0-1; second phase (2):
// target rows p0..gamma-1, then draft rows p0..gamma-1.
__device__ inline uint32_t group_stream_row(const Params& P, int phase, uint32_t j) {
    const uint32_t gamma = static_cast<uint32_t>(P.gamma), nt = gamma + 1u, p0 = static_cast<uint32_t>(P.p0);
    if (phase == 1) return j < p0 ? j : nt + (j - p0);
    if (phase == 2) return j < gamma - p0 ? p0 + j : nt + p0 + (j - (gamma - p0));
    return P.defer && j >= gamma ? j + 1u : j;
}

// Row j of group g: target rows 0..gamma, then draft rows 0..gamma-1.
template <int DT>
__device__ inline const char* group_row(const Params& P, uint32_t g, uint32_t j) {
    const uint32_t nt = static_cast<uint32_t>(P.gamma) + 1u;
    if (j < nt) return row_at<DT>(P.tgt, (static_cast<int64_t>(g) * nt + j) * P.V);
    return row_at<DT>(P.dft, (static_cast<int64_t>(g) * P.gamma + (j - nt)) * P.V);
}


// --------------------------------------------------------------------------
// Waits and decision words
// --------------------------------------------------------------------------
// What the decision words of positions 0..i-1 of sequence b say (one
// wavefront, lane j reads position j): kLive if all were accepted, kStopped if
// the first that was not is a rejection or an unusable row, kUnknown if that
// one is still pending.
// (Split in two so that the load can be issued early: lane j < i loads
// position j's word, state_of reads the loaded words.)
__device__ inline uint64_t decision_word(const Params& P, int32_t b, int32_t i, int lane) {
    return lane < i ? cld64(P.dec + static_cast<int64_t>(b) * (P.gamma + 1) + lane) : 0ull;
}
__device__ inline int state_of(const Params& P, uint64_t w, int32_t i, int lane) {
    uint32_t st = kAcc;
    if (lane < i) st = static_cast<uint32_t>(w >> 32) == P.epoch ? static_cast<uint32_t>(w & 3u) : kPending;
    const uint64_t open = __ballot(st != kAcc);
    if (!open) return kLive;
    const int f = __ffsll(static_cast<unsigned long long>(open)) - 1;
    return __shfl(static_cast<int>(st), f, kWave) == static_cast<int>(kPending) ? kUnknown : kStopped;
}
__device__ inline int sequence_state(const Params& P, int32_t b, int32_t i, int lane) {
    return state_of(P, decision_word(P, b, i, lane), i, lane);
}
// `s` is the state from an earlier read (kUnknown: read again until known).
// If the bound runs out, the sticky error word is set and `late` raised, and
// the read goes on (drains) up to kWaitTicks, so that the caller still learns
// whether its position ends the sequence; kTimedOut if that runs out too.
__device__ inline int wait_sequence_state(const Params& P, int32_t b, int32_t i, int lane, int s, bool& late) {
    late = false;
    if (s != kUnknown) return s;
    auto known = [&] {
        s = sequence_state(P, b, i, lane);
        return s != kUnknown;
    };
    if (spin_until(known, P.wait)) return s;
    late = true;
    if (lane == 0) cst(P.err, 1u);
    return spin_until(known, kWaitTicks) ? s : kTimedOut;
}
__device__ inline void publish(const Params& P, int32_t b, int32_t i, uint32_t status) {
    cst64(P.dec + static_cast<int64_t>(b) * (P.gamma + 1) + i, (static_cast<uint64_t>(P.epoch) << 32) | status);
}

// The outputs of sequence b when it stops at position k (lane j writes
// out_tokens[b, j]; x = draft token j): n = k, the k accepted draft tokens,
// -1 after k; the token at k itself is written by whoever computes it. With
// invalid, n = -1 and the whole row -1.
__device__ inline void write_outputs(const Params& P, int32_t b, int32_t k, bool invalid, int32_t x, int lane) {
    const int nt = P.gamma + 1;
    if (lane < nt && (invalid || lane != k))
        cst(P.out_tokens + static_cast<int64_t>(b) * nt + lane, (!invalid && lane < k) ? x : -1);
    if (lane == 0) cst(P.out_n + b, invalid ? -1 : k);
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

// Sum of 2^(fl(x*c - R)) over N chunks in two fp32 accumulators (no maximum).
template <int DT, bool VEC, int N>
__device__ inline float group_exp_sum(const typename Chunk<DT, VEC>::Raw* raw, float c, float R) {
    using C = Chunk<DT, VEC>;
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int u = 0; u < N; ++u) {
        float x[C::EPL];
        C::expand(raw[u], x);
#pragma unroll
        for (int v = 0; v < C::EPL; ++v) {
            const float e = __builtin_amdgcn_exp2f(fmaf(x[v], c, -R));
            if (v & 1) a1 += e;
            else a0 += e;
        }
    }
    return a0 + a1;
}

// The same sum and, beside it, the sum of 2^t * t (t = fl(x*c - R)), for the
// entropy (a zero mass contributes zero, also where t = -inf).
template <int DT, bool VEC, int N>
__device__ inline void group_exp_tsum(const typename Chunk<DT, VEC>::Raw* raw, float c, float R, float& sum,
                                      float& tsum) {
    using C = Chunk<DT, VEC>;
    float a0 = 0.0f, a1 = 0.0f, b0 = 0.0f, b1 = 0.0f;
#pragma unroll
    for (int u = 0; u < N; ++u) {
        float x[C::EPL];
        C::expand(raw[u], x);
#pragma unroll
        for (int v = 0; v < C::EPL; ++v) {
            const float t = fmaf(x[v], c, -R);
            const float e = __builtin_amdgcn_exp2f(t);
            const float et = e > 0.0f ? e * t : 0.0f;
            if (v & 1) {
                a1 += e;
                b1 += et;
            } else {
                a0 += e;
                b0 += et;
            }
        }
    }
    sum = a0 + a1;
    tsum = b0 + b1;
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
    int64_t slot;  // (unit*2 + j)*maxp + k
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
    uint32_t skip;  // (second phase: the sequence stopped within the first)
};

// Statistics of one wavefront's chunk range [wl*cpw, (wl+1)*cpw) of the unit's
// (group-major: the group's) concatenated rows: one partial per row piece, for
// slot (unit*2 + j)*maxp + k (group-major: (g*rps + j)*maxp + k),
// k = wl minus the first wavefront touching row j. The piece that ends a row
// also covers the row's unused slots (a row spans maxp - 1 or maxp
// wavefronts), which are written with neutral values, so folds read every
// slot. Returns the number of pieces placed in `out` (lane 0 writes them).
template <int DT, bool VEC, int MODE, bool GROUP = false, bool NT = true>
__device__ inline int stats_wave(const Params& P, const Role& U, uint32_t wl, int lane, Piece* out) {
    int npieces = 0;
    using C = Chunk<DT, VEC>;
    using Raw = typename C::Raw;
    using Lane = typename std::conditional<MODE == kGreedy, ArgLane, SoftLane>::type;
    const float c = P.c32;
    const bool watch = !GROUP && MODE != kRows && P.skip && U.i > 0;
    const uint32_t nchunk = static_cast<uint32_t>(P.nchunk);
    const uint32_t cpw = static_cast<uint32_t>(GROUP && U.i == 2 ? P.cpw2 : P.cpw);
    const uint32_t total = static_cast<uint32_t>(U.rows) * nchunk;
    uint32_t cc = wl * cpw;
    const uint32_t c_end = cc + cpw < total ? cc + cpw : total;
    uint32_t j = cc / nchunk;
    uint32_t first = j * nchunk;
    int32_t k = static_cast<int32_t>(wl - first / cpw);
    while (cc < c_end) {
        const uint32_t ce = first + nchunk < c_end ? first + nchunk : c_end;
        const uint32_t jr = GROUP ? group_stream_row(P, U.i, j) : j;
        const char* row = GROUP ? group_row<DT>(P, U.unit, jr) : unit_row<DT, MODE>(P, U, static_cast<int32_t>(j));
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
            for (int u = 0; u < kUnroll; ++u) q[u] = C::template load_full<NT>(row, c0 + gi * kUnroll + u, lane);
            __builtin_amdgcn_sched_barrier(0);
        };
        auto load_last = [&](Raw* q, int64_t gi) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) q[u] = C::template load_clamped<NT>(row, c0 + gi * kUnroll + u, c_last, lane, P.V);
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
                // early stop: the sequence's earlier decision words are read
                // with this round's loads; if it stopped meanwhile, the rest of
                // the range is left unread (the wavefront returns no pieces)
                const uint64_t wd = watch ? decision_word(P, U.b, U.i, lane) : 0ull;
                load(qb, gi);
                eat(qa, gi - 1);
                load(qa, gi + 1);
                eat(qb, gi);
                if (watch && state_of(P, wd, U.i, lane) == kStopped) return 0;
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
        pc.slot = (GROUP ? (static_cast<int64_t>(U.unit) * P.rps + jr) * P.maxp
                         : slot_base(P, U.unit, static_cast<int32_t>(j))) + k;
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
// Folding partials. A row's partials (m, r, s) combine exactly with ldexp onto
// the larger reference r; the row's sum in exp((x - max)/T) units is
// s * 2^(r - max*c), the exponent formed exactly in fp64. Argmax partials
// combine as (value desc, index asc); a NaN marks the row.
// --------------------------------------------------------------------------

struct RowPart {
    float m;
    float r;
    double s;
};
__device__ inline RowPart row_none() { return RowPart{-INFINITY, kRUnset, 0.0}; }
__device__ inline RowPart fold(const RowPart& a, const RowPart& b) {
    const float r = fmaxf(a.r, b.r);
    return RowPart{fmaxf(a.m, b.m), r, rebase(a.s, a.r, r) + rebase(b.s, b.r, r)};
}
__device__ inline double row_sum(const RowPart& f, float c32) {
    return f.s * exp2(static_cast<double>(f.r) - static_cast<double>(f.m) * static_cast<double>(c32));
}
__device__ inline bool usable(float M, double S) { return isfinite(M) && isfinite(S) && S > 0.0; }
__device__ inline RowPart wave_fold_rows(RowPart f) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const RowPart g{__shfl_xor(f.m, o, kWave), __shfl_xor(f.r, o, kWave), __shfl_xor(f.s, o, kWave)};
        f = fold(f, g);
    }
    return f;
}

struct ArgPart {
    float m;
    int32_t at;
};
__device__ inline ArgPart fold_arg(const ArgPart& a, const ArgPart& b) {
    const bool nan = a.m != a.m || b.m != b.m;
    const bool tb = b.m > a.m || (b.m == a.m && b.at < a.at);
    ArgPart o;
    o.m = nan ? NAN : (tb ? b.m : a.m);
    o.at = tb ? b.at : a.at;
    return o;
}

// The unit's rows folded from their slots by one wavefront (lane k takes slots
// k, k + 64, ...; both rows' loads are issued together), the same in every
// wavefront that folds them.
__device__ inline void merge_rows(const Params& P, uint32_t unit, int rows, int lane, RowPart* out) {
    RowPart f0 = row_none(), f1 = row_none();
    for (int k = lane; k < P.maxp; k += kWave) {
        const int64_t a = slot_base(P, unit, 0) + k, b = slot_base(P, unit, 1) + k;
        const float m0 = cld(P.part_m + a), r0 = cld(P.part_r + a);
        const double s0 = cld(P.part_s + a);
        float m1 = -INFINITY, r1 = kRUnset;
        double s1 = 0.0;
        if (rows > 1) {
            m1 = cld(P.part_m + b);
            r1 = cld(P.part_r + b);
            s1 = cld(P.part_s + b);
        }
        f0 = fold(f0, RowPart{m0, r0, s0});
        f1 = fold(f1, RowPart{m1, r1, s1});
    }
    out[0] = wave_fold_rows(f0);
    out[1] = wave_fold_rows(f1);
}
__device__ inline ArgPart merge_arg(const Params& P, uint32_t unit, int lane) {
    ArgPart f{-INFINITY, INT32_MAX};
    for (int k = lane; k < P.maxp; k += kWave) {
        const int64_t a = slot_base(P, unit, 0) + k;
        f = fold_arg(f, ArgPart{cld(P.part_m + a), cld(P.part_i + a)});
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) f = fold_arg(f, ArgPart{__shfl_xor(f.m, o, kWave), __shfl_xor(f.at, o, kWave)});
    return f;
}

// Makes the compiler forget what it knows about a held chunk, so values
// expanded from it in one pass are formed again in the next rather than kept
// live (which would need 128 more registers for bf16).
__device__ inline void opaque(uint4& r) { asm volatile("" : "+v"(r.x), "+v"(r.y), "+v"(r.z), "+v"(r.w)); }
__device__ inline void opaque(float4& r) { asm volatile("" : "+v"(r.x), "+v"(r.y), "+v"(r.z), "+v"(r.w)); }


// --------------------------------------------------------------------------
// Registers: N chunk slots starting at chunk c0 of a row. Chunks before the
// row's last are loaded whole; the last one from valid addresses only (its
// elements at or beyond V are set to -inf by mask_slots once loaded); slots
// past the row read as -inf without a load. All loads are issued before any
// is consumed.
// --------------------------------------------------------------------------
template <int DT, bool VEC, int N, bool NT = true>
__device__ inline void load_slots(typename Chunk<DT, VEC>::Raw* q, const char* row, int64_t c0, int32_t nchunk,
                                  int32_t V, int lane) {
    using C = Chunk<DT, VEC>;
    const int64_t c_last = nchunk - 1;
#pragma unroll
    for (int u = 0; u < N; ++u) {
        const int64_t c = c0 + u;
        if (c < c_last) q[u] = C::template load_full<NT>(row, c, lane);
        else if (c == c_last) q[u] = C::template load_clamped<NT>(row, c, c_last, lane, V);
        else q[u] = C::blank();
    }
}
template <int DT, bool VEC, int N>
__device__ inline void mask_slots(typename Chunk<DT, VEC>::Raw* q, int64_t c0, int32_t nchunk, int32_t V, int lane) {
    using C = Chunk<DT, VEC>;
    const int64_t c_last = nchunk - 1;
#pragma unroll
    for (int u = 0; u < N; ++u)
        if (c0 + u == c_last) q[u] = C::mask(q[u], c_last, c_last, lane, V);
}

// --------------------------------------------------------------------------
// Draw masses in t units. With e_j = 2^(fl(x_j*c) - mc) for the target (p) and
// draft (q) rows, p_j = e_pj * scale_p and q_j = e_qj * scale_q (scale =
// 2^(mc - m*c)/S). Then max(0, p_j - q_j) = scale_p * t_j with
// t_j = max(0, e_pj - rho*e_qj), rho = scale_q/scale_p. t_j is formed in fp32
// with rho split into an fp32 pair (hi + lo, two FMAs), so the product keeps
// about 48 bits; every sum over elements is fp64. The inverse-CDF draw is
// invariant to the common factor; drawing from p, t_j = e_pj.
// --------------------------------------------------------------------------
struct MassRow {
    float mcp, mcq;  // fl(max*c) of the target / draft row
    float rhi, rlo;  // rho = rhi + rlo
    float c32;
    int32_t has_q;   // 0: masses of p alone
};
__device__ inline float elem_mass(float xp, float xq, const MassRow& m) {
    const float ep = __builtin_amdgcn_exp2f(fmaf(xp, m.c32, -m.mcp));
    if (!m.has_q) return ep;
    const float eq = __builtin_amdgcn_exp2f(fmaf(xq, m.c32, -m.mcq));
    return fmaxf(0.0f, fmaf(-eq, m.rlo, fmaf(-eq, m.rhi, ep)));
}

// A wavefront's held pair (target chunks in slots [0, kPairCw), the draft's
// same chunks in [kPairCw, 2*kPairCw)) is visited in ascending index order as
// tiles: one chunk per tile on the vector path (each lane's EPL consecutive
// elements), one element per lane per tile on the scalar path (element v of
// every lane, then v + 1). A tile's lane mass is the fp64 sum of its elements'
// masses in index order; tile totals are wave scans of the lane masses, added
// in tile order. wave_mass and wave_draw form these sums identically.
template <int DT, bool VEC>
struct Tiles {
    using C = Chunk<DT, VEC>;
    static constexpr int PER_CHUNK = VEC ? 1 : C::EPL;  // tiles per chunk
    static constexpr int EPT = VEC ? C::EPL : 1;        // elements per lane per tile
};

template <int DT, bool VEC>
__device__ inline double wave_mass(typename Chunk<DT, VEC>::Raw* q, const MassRow& m) {
    using C = Chunk<DT, VEC>;
    using T = Tiles<DT, VEC>;
#pragma unroll
    for (int u = 0; u < kHold; ++u) opaque(q[u]);
    double base = 0.0;
#pragma unroll
    for (int u = 0; u < kPairCw; ++u) {
        float xp[C::EPL], xq[C::EPL];
        C::expand(q[u], xp);
        C::expand(q[kPairCw + u], xq);
#pragma unroll
        for (int t = 0; t < T::PER_CHUNK; ++t) {
            double lm = 0.0;
#pragma unroll
            for (int e = 0; e < T::EPT; ++e) {
                const int v = VEC ? e : t;
                lm += static_cast<double>(elem_mass(xp[v], xq[v], m));
            }
            base += wave_sum(lm);
        }
    }
    return base;
}

// The element of this wavefront's range where the cumulative mass, starting
// at `base`, first exceeds `target` (smallest index); if rounding leaves no
// crossing, the last element with mass; -1 if the range has none.
template <int DT, bool VEC>
__device__ inline int32_t wave_draw(typename Chunk<DT, VEC>::Raw* q, const MassRow& m, int64_t c0,
                                    double base, double target, int lane) {
    using C = Chunk<DT, VEC>;
    using T = Tiles<DT, VEC>;
#pragma unroll
    for (int u = 0; u < kHold; ++u) opaque(q[u]);
    int32_t last = -1;
#pragma unroll
    for (int u = 0; u < kPairCw; ++u) {
        float xp[C::EPL], xq[C::EPL];
        C::expand(q[u], xp);
        C::expand(q[kPairCw + u], xq);
#pragma unroll
        for (int t = 0; t < T::PER_CHUNK; ++t) {
            float mv[T::EPT];
            double lm = 0.0;
            int32_t mylast = -1;
#pragma unroll
            for (int e = 0; e < T::EPT; ++e) {
                const int v = VEC ? e : t;
                mv[e] = elem_mass(xp[v], xq[v], m);
                lm += static_cast<double>(mv[e]);
                if (mv[e] > 0.0f) mylast = static_cast<int32_t>(C::index_of(c0 + u, lane, v));
            }
            const double incl = base + wave_scan_incl(lm);
            const double prev = lane_before(incl);
            const double excl = lane == 0 ? base : prev;
            const uint64_t hit = __ballot(lm > 0.0 && excl <= target && target < incl);
            if (hit) {
                const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
                int32_t pick = -1;
                if (lane == l) {
                    double run = excl;
#pragma unroll
                    for (int e = 0; e < T::EPT; ++e) {
                        run += static_cast<double>(mv[e]);
                        if (pick < 0 && mv[e] > 0.0f && run > target)
                            pick = static_cast<int32_t>(C::index_of(c0 + u, lane, VEC ? e : t));
                    }
                    if (pick < 0) pick = mylast;
                }
                return __shfl(pick, l, kWave);
            }
            const uint64_t mass = __ballot(mylast >= 0);
            if (mass) last = __shfl(mylast, 63 - __clzll(static_cast<unsigned long long>(mass)), kWave);
            base = lane_f64(incl, kWave - 1);
        }
    }
    return last;
}

// --------------------------------------------------------------------------
// The unit's last block
// --------------------------------------------------------------------------
// Counts the calling wavefront in at a unit counter once its coherent stores
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

// Draw record of sequence b: words 0..5 each carry the call's epoch in their
// high half, so a reader that sees the epoch in all six has the whole record
// (one round trip, no separate tag): kind << 8 | k, then mcp, mcq, rhi, rlo
// and scale_p (as fp32). Its ticket counters are zeroed and complete before
// any word goes out (lane 0 writes).
constexpr int kRecFields = 6;
__device__ inline uint64_t tagged(const Params& P, uint32_t v) { return (static_cast<uint64_t>(P.epoch) << 32) | v; }
// The draw's two ticket counters live beside its record: the record's writer
// sets them to zero before the tag goes out and no block touches them before
// seeing the tag, so they need no clearing between calls.
__device__ inline uint32_t* claim_counter(const Params& P, int32_t b) {
    return reinterpret_cast<uint32_t*>(P.rec + static_cast<int64_t>(b) * kRecWords + kClaimWord);
}
__device__ inline uint32_t* piece_counter(const Params& P, int32_t b) {
    return reinterpret_cast<uint32_t*>(P.rec + static_cast<int64_t>(b) * kRecWords + kPieceWord);
}

__device__ inline void write_record(const Params& P, int32_t b, uint32_t kind, int32_t k, const MassRow& m,
                                    double scale_p) {
    uint64_t* r = P.rec + static_cast<int64_t>(b) * kRecWords;
    cst(claim_counter(P, b), 0u);
    cst(piece_counter(P, b), 0u);
    complete_before();
    cst64(r, tagged(P, (kind << 8) | static_cast<uint32_t>(k)));
    cst64(r + 1, tagged(P, __float_as_uint(m.mcp)));
    cst64(r + 2, tagged(P, __float_as_uint(m.mcq)));
    cst64(r + 3, tagged(P, __float_as_uint(m.rhi)));
    cst64(r + 4, tagged(P, __float_as_uint(m.rlo)));
    cst64(r + 5, tagged(P, __float_as_uint(static_cast<float>(scale_p))));
}

// T > 0: the accept step of position i from the unit's folded rows (one
// wavefront). The bonus unit (i == gamma) only checks that its row is usable.
// The acceptance probability alpha = min(1, p/q) of a draft token from its
// exponents ep = (l_t - m_t)*c and eq = (l_d - m_d)*c (both <= 0) and the two
// rows' sums (both >= 1): where neither p = 2^ep/st nor q = 2^eq/sd can be
// zero or subnormal, alpha = min(1, 2^(ep - eq) * sd/st) (one exp2, one
// division); otherwise p and q are formed first and the zero rules apply
// (p = 0: 0; q = 0: 1).
__device__ inline double accept_prob(double ep, double st, double eq, double sd) {
    if (ep > -900.0 && eq > -900.0) return fmin(1.0, exp2(ep - eq) * (sd / st));
    const double p = exp2(ep) / st, q = exp2(eq) / sd;
    return p == 0.0 ? 0.0 : (q == 0.0 ? 1.0 : fmin(1.0, p / q));
}
// The accept test u < alpha with alpha = accept_prob(...): first in fp32, the
// exponent ep - eq split exactly (fp64) into an integer n and a fraction in
// [-1/2, 1/2], so that alpha comes within about 5e-7 (relative) of its fp64
// value; that settles every u farther than 1e-5 (relative) from alpha, with
// the fp64 test's outcome. The rest, and whatever the fp32 form cannot hold,
// take the fp64 test.
__device__ inline bool accept_test(double u, double ep, double st, double eq, double sd) {
    if (ep > -900.0 && eq > -900.0) {
        const double a = ep - eq;
        const double n = rint(a);
        if (fabs(n) < 100.0) {
            const float r = ldexpf(__builtin_amdgcn_exp2f(static_cast<float>(a - n)), static_cast<int>(n)) *
                            (static_cast<float>(sd) / static_cast<float>(st));
            const double alpha = static_cast<double>(fminf(1.0f, r));
            if (u < alpha * (1.0 - 1e-5)) return true;
            if (u > alpha * (1.0 + 1e-5)) return false;
        }
    }
    return u < accept_prob(ep, st, eq, sd);
}

template <int DT>
__device__ inline void decide_sample(const Params& P, const Role& U, int lane) {
    const int32_t gamma = P.gamma, V = P.V, nt = gamma + 1;
    const bool pair = U.i < gamma;
    int32_t xj = 0;
    if (lane < gamma) xj = P.tokens[static_cast<int64_t>(U.b) * gamma + lane];
    const int32_t x = pair ? __shfl(xj, U.i, kWave) : 0;
    const bool tok_ok = x >= 0 && x < V;
    // the accept uniform does not depend on the statistics: drawn before the loads
    const double u = pair ? philox_uniform(P.seed, static_cast<uint32_t>(U.b + P.b_offset), static_cast<uint32_t>(U.i), 0u)
                          : 0.0;
    float lt = 0.0f, ld = 0.0f;
    if (pair) {
        lt = cld(P.tok_l + static_cast<int64_t>(U.unit) * 2);
        ld = cld(P.tok_l + static_cast<int64_t>(U.unit) * 2 + 1);
    }
    // the earlier positions' words are read with the unit's slots (one round
    // trip); they are needed only if position i ends the sequence
    const uint64_t wd = decision_word(P, U.b, U.i, lane);
    RowPart rs[2];
    merge_rows(P, U.unit, U.rows, lane, rs);
    const float c = P.c32;
    const double cd = static_cast<double>(c);
    const float Mt = rs[0].m, Md = rs[1].m;
    const double st = row_sum(rs[0], c), sd = row_sum(rs[1], c);
    const bool ut = usable(Mt, st), ud = usable(Md, sd);
    uint32_t status = kAcc;
    double p = NAN, qv = NAN;
    if (pair) {
        if (!ut || !ud || !tok_ok) {
            status = kBad;
        } else {
            const double ep = (static_cast<double>(lt) - static_cast<double>(Mt)) * cd;
            const double eq = (static_cast<double>(ld) - static_cast<double>(Md)) * cd;
            status = accept_test(u, ep, st, eq, sd) ? kAcc : kRej;
            if (P.dbg_p || P.dbg_q) {
                p = exp2(ep) / st;
                qv = exp2(eq) / sd;
            }
        }
    } else if (!ut) {
        status = kBad;
    }
    if (lane == 0) {
        const int64_t R = 2 * gamma + 1;
        if (P.dbg_row_max) P.dbg_row_max[U.b * R + U.i] = Mt;
        if (P.dbg_row_sumexp) P.dbg_row_sumexp[U.b * R + U.i] = st;
        if (pair) {
            if (P.dbg_row_max) P.dbg_row_max[U.b * R + nt + U.i] = Md;
            if (P.dbg_row_sumexp) P.dbg_row_sumexp[U.b * R + nt + U.i] = sd;
            if (P.dbg_p) P.dbg_p[static_cast<int64_t>(U.b) * gamma + U.i] = p;
            if (P.dbg_q) P.dbg_q[static_cast<int64_t>(U.b) * gamma + U.i] = qv;
        }
    }
    // every position's outcome is published at once; only the position that
    // ends the sequence (its first non-accepted one, or the bonus row) waits
    // for the earlier positions' outcomes
    if (pair && lane == 0) publish(P, U.b, U.i, status);
    if (pair && status == kAcc) return;
    bool late = false;
    const int state = U.i > 0 ? wait_sequence_state(P, U.b, U.i, lane, state_of(P, wd, U.i, lane), late) : kLive;
    if (state == kStopped) return;
    MassRow mr;
    mr.c32 = c;
    mr.has_q = pair ? 1 : 0;
    mr.mcp = Mt * c;
    const double scale_p = exp2(static_cast<double>(mr.mcp) - static_cast<double>(Mt) * cd) / st;
    mr.mcq = pair ? Md * c : 0.0f;
    const double rho = pair ? exp2((static_cast<double>(mr.mcq) - static_cast<double>(Md) * cd) -
                                   (static_cast<double>(mr.mcp) - static_cast<double>(Mt) * cd)) * (st / sd)
                            : 0.0;
    mr.rhi = static_cast<float>(rho);
    mr.rlo = static_cast<float>(rho - static_cast<double>(mr.rhi));
    if (state == kTimedOut || late) {
        // this position ends the sequence, but its wait for the earlier
        // positions ran out: the sequence is reported invalid
        write_outputs(P, U.b, U.i, true, xj, lane);
        if (lane == 0) write_record(P, U.b, kNoDraw, U.i, mr, scale_p);
        return;
    }
    if (status == kBad) {
        write_outputs(P, U.b, U.i, true, xj, lane);
        if (lane == 0) {
            if (P.dbg_z) P.dbg_z[U.b] = NAN;
            write_record(P, U.b, kNoDraw, U.i, mr, scale_p);
        }
        return;
    }
    // position i ends the sequence: a rejection (draw from the residual) or the
    // bonus row after gamma acceptances (draw from p); the token is drawn by the
    // sequence's residual blocks
    write_outputs(P, U.b, U.i, false, xj, lane);
    if (lane == 0) {
        write_record(P, U.b, pair ? kDrawResidual : kDrawP, U.i, mr, scale_p);
    }
}

// T == 0: the greedy step of position i (one wavefront): accept while the
// draft token is the row's argmax (lowest index on ties), else emit the
// argmax; at the bonus row (all gamma accepted) emit its argmax.
__device__ inline void decide_greedy(const Params& P, const Role& U, int lane) {
    const int32_t gamma = P.gamma, V = P.V, nt = gamma + 1;
    int32_t xj = 0;
    if (lane < gamma) xj = P.tokens[static_cast<int64_t>(U.b) * gamma + lane];
    const ArgPart f = merge_arg(P, U.unit, lane);
    if (lane == 0) {
        if (P.dbg_row_max) P.dbg_row_max[U.b * static_cast<int64_t>(2 * gamma + 1) + U.i] = f.m;
        if (P.dbg_argmax) P.dbg_argmax[static_cast<int64_t>(U.b) * nt + U.i] = f.at;
    }
    const bool ut = isfinite(f.m);
    const uint64_t wd = decision_word(P, U.b, U.i, lane);
    uint32_t status;
    if (U.i < gamma) {
        const int32_t x = __shfl(xj, U.i, kWave);
        status = (!ut || !(x >= 0 && x < V)) ? kBad : (x == f.at ? kAcc : kRej);
        if (lane == 0) publish(P, U.b, U.i, status);  // at once; see decide_sample
    } else {
        status = ut ? kRej : kBad;  // the bonus row ends the sequence either way
    }
    if (status == kAcc) return;
    bool late = false;
    const int state = U.i > 0 ? wait_sequence_state(P, U.b, U.i, lane, state_of(P, wd, U.i, lane), late) : kLive;
    if (state == kStopped) return;
    if (state == kTimedOut || late) {  // ends the sequence, but its wait ran out: reported invalid
        write_outputs(P, U.b, U.i, true, xj, lane);
        return;
    }
    write_outputs(P, U.b, U.i, status == kBad, xj, lane);
    if (status != kBad && lane == 0) cst(P.out_tokens + static_cast<int64_t>(U.b) * nt + U.i, f.at);
}

// Row statistics: the row's max and sum (one wavefront).
__device__ inline void finish_rows(const Params& P, const Role& U, int lane) {
    RowPart rs[2];
    merge_rows(P, U.unit, 1, lane, rs);
    if (lane == 0) {
        const double s = row_sum(rs[0], P.c32);
        cst(P.rows_max + U.b, rs[0].m);
        cst(P.rows_sumexp + U.b, usable(rs[0].m, s) ? s : static_cast<double>(NAN));
        if (P.tree_done) {  // the tree's closing wavefront waits for all 2*tree_n of its rows
            complete_before();
            const int64_t r = U.b < P.rows_split ? U.b : U.b - P.rows_split;
            (void)__hip_atomic_fetch_add(P.tree_done + (r / P.tree_n) * kSyncStride, 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// A statistics block: each wavefront streams its chunk range (nothing if its
// sequence already stopped), the block's last wavefront writes the block's
// pieces and counts the block in, and the unit's last block decides.
// --------------------------------------------------------------------------
// T > 0: the draw of a sequence that stopped at position k. Its stopping rows
// are split into nbr pieces of kWavesPerBlock*kPairCw chunks of each row; a
// block claims a piece (an atomic ticket), loads it into registers, stores one
// mass per wavefront and counts the piece in; the block that counts in the
// last piece draws the token: scans of the per-wavefront masses give Z and the
// wavefront holding u*Z, whose chunks it loads again and scans. Blocks of the
// sequence's later positions (which the early stop leaves idle) and the
// grid's closing blocks claim pieces until none is left.
// --------------------------------------------------------------------------
struct DrawInfo {
    int32_t kind;  // kNoDraw, kDrawResidual or kDrawP
    int32_t k;     // stopping position
    MassRow mr;
    double scale_p;
};

// One read of sequence b's draw record (one wavefront): false until all of
// its words carry this call's epoch.
__device__ inline bool read_record(const Params& P, int32_t b, int lane, DrawInfo& d) {
    const uint64_t* r = P.rec + static_cast<int64_t>(b) * kRecWords;
    const uint64_t v = lane < kRecFields ? cld64(r + lane) : tagged(P, 0u);
    if (__ballot(static_cast<uint32_t>(v >> 32) != P.epoch) != 0) return false;
    const uint32_t x = static_cast<uint32_t>(v);
    const uint32_t w0 = __shfl(x, 0, kWave);
    d.kind = static_cast<int32_t>((w0 >> 8) & 0xFFu);
    d.k = static_cast<int32_t>(w0 & 0xFFu);
    d.mr.mcp = __uint_as_float(__shfl(x, 1, kWave));
    d.mr.mcq = __uint_as_float(__shfl(x, 2, kWave));
    d.mr.rhi = __uint_as_float(__shfl(x, 3, kWave));
    d.mr.rlo = __uint_as_float(__shfl(x, 4, kWave));
    d.scale_p = static_cast<double>(__uint_as_float(__shfl(x, 5, kWave)));
    d.mr.c32 = P.c32;
    d.mr.has_q = d.kind == kDrawResidual ? 1 : 0;
    return true;
}

// Wavefront `gw` of the stopping rows: chunks [gw*kPairCw, (gw+1)*kPairCw) of
// the target row k (slots [0, kPairCw)) and of the draft row k when has_q.
template <int DT, bool VEC>
__device__ inline void load_wave_chunks(const Params& P, int32_t b, int32_t k, bool has_q, int64_t gw,
                                        typename Chunk<DT, VEC>::Raw* q, int lane) {
    using C = Chunk<DT, VEC>;
    const int64_t c0 = gw * kPairCw;
    const char* trow = row_at<DT>(P.tgt, (static_cast<int64_t>(b) * (P.gamma + 1) + k) * P.V);
    load_slots<DT, VEC, kPairCw>(q, trow, c0, P.nchunk, P.V, lane);
    if (has_q) {
        const char* drow = row_at<DT>(P.dft, (static_cast<int64_t>(b) * P.gamma + k) * P.V);
        load_slots<DT, VEC, kPairCw>(q + kPairCw, drow, c0, P.nchunk, P.V, lane);
    } else {
#pragma unroll
        for (int u = kPairCw; u < kHold; ++u) q[u] = C::blank();
    }
    mask_slots<DT, VEC, kPairCw>(q, c0, P.nchunk, P.V, lane);
    if (has_q) mask_slots<DT, VEC, kPairCw>(q + kPairCw, c0, P.nchunk, P.V, lane);
}

// Total of m[0, n) in the order the search below accumulates it.
__device__ inline double scan_total(const double* m, int32_t n, int lane) {
    double base = 0.0;
    for (int32_t t0 = 0; t0 < n; t0 += kWave) {
        const double v = t0 + lane < n ? cld(m + t0 + lane) : 0.0;
        base += lane_f64(wave_scan_incl(v), kWave - 1);
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
        const double incl = base + wave_scan_incl(v);
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


// The token of sequence b, by the block that counted in its last piece: Z and
// the wavefront holding u*Z from the per-wavefront masses (wavefront 0), then
// that wavefront's chunks scanned again. A rejected row whose residual rounds
// to zero draws from p_k instead: the block recomputes every wavefront's p
// mass first (never on the common path).
template <int DT, bool VEC>
__device__ inline void draw_sequence(const Params& P, int32_t b, DrawInfo d, int w, int lane) {
    using Raw = typename Chunk<DT, VEC>::Raw;
    __shared__ double s_z;
    const int32_t n = P.nbr * kWavesPerBlock;
    double* m = P.msum + static_cast<int64_t>(b) * n;
    if (w == 0) {
        after_complete();
        const double z = scan_total(m, n, lane);
        if (lane == 0) {
            s_z = z;
            if (P.dbg_z) P.dbg_z[b] = z * d.scale_p;
        }
    }
    __syncthreads();
    double z = s_z;
    if (d.mr.has_q && !(z > 0.0)) {
        d.mr.has_q = 0;
        for (int32_t gw = w; gw < n; gw += kWavesPerBlock) {
            Raw q[kHold];
            load_wave_chunks<DT, VEC>(P, b, d.k, false, gw, q, lane);
            const double wm = wave_mass<DT, VEC>(q, d.mr);
            if (lane == 0) cst(m + gw, wm);
        }
        complete_before();
        __syncthreads();
        if (w == 0) {
            after_complete();
            const double zp = scan_total(m, n, lane);
            if (lane == 0) s_z = zp;
        }
        __syncthreads();
        z = s_z;
    }
    if (w != 0) return;
    const int32_t nt = P.gamma + 1;
    const double u = philox_uniform(P.seed, static_cast<uint32_t>(b + P.b_offset), static_cast<uint32_t>(d.k), 1u);
    const double target = u * z;
    double before = 0.0;
    const int32_t sel = scan_find(m, n, target, lane, before);
    int32_t tok = -1;  // no mass at all (cannot happen for a usable row): keep the output defined
    if (sel >= 0) {
        Raw q[kHold];
        load_wave_chunks<DT, VEC>(P, b, d.k, d.mr.has_q != 0, sel, q, lane);
        tok = wave_draw<DT, VEC>(q, d.mr, static_cast<int64_t>(sel) * kPairCw, before, target, lane);
    }
    if (lane == 0) cst(P.out_tokens + static_cast<int64_t>(b) * nt + d.k, tok);
}

// Claims pieces of sequence b's stopping rows until none is left (every
// thread of the block; d.kind is a draw).
template <int DT, bool VEC>
__device__ inline void claim_pieces(const Params& P, int32_t b, const DrawInfo& d) {
    using Raw = typename Chunk<DT, VEC>::Raw;
    __shared__ uint32_t s_piece, s_last;
    const int lane = static_cast<int>(threadIdx.x & (kWave - 1));
    const int w = static_cast<int>(__builtin_amdgcn_readfirstlane(threadIdx.x / kWave));
    const uint32_t np = static_cast<uint32_t>(P.nbr);
    uint32_t* claim = claim_counter(P, b);
    uint32_t* done = piece_counter(P, b);
    for (;;) {
        if (threadIdx.x == 0) s_piece = __hip_atomic_fetch_add(claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const uint32_t piece = s_piece;
        if (piece >= np) return;
        Raw q[kHold];
        const int64_t gw = static_cast<int64_t>(piece) * kWavesPerBlock + w;
        load_wave_chunks<DT, VEC>(P, b, d.k, d.mr.has_q != 0, gw, q, lane);
        const double wm = wave_mass<DT, VEC>(q, d.mr);
        if (lane == 0) cst(P.msum + static_cast<int64_t>(b) * np * kWavesPerBlock + gw, wm);
        complete_before();
        __syncthreads();
        if (threadIdx.x == 0)
            s_last = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == np ? 1u : 0u;
        __syncthreads();
        if (s_last) draw_sequence<DT, VEC>(P, b, d, w, lane);
        __syncthreads();
    }
}

// A closing block of sequence b: waits for the draw record, then claims.
template <int DT, bool VEC>
__device__ inline void resid_block(const Params& P, const Role& U) {
    __shared__ int32_t s_ok;
    __shared__ DrawInfo s_d;
    const int lane = static_cast<int>(threadIdx.x & (kWave - 1));
    const int w = static_cast<int>(__builtin_amdgcn_readfirstlane(threadIdx.x / kWave));
    const int32_t b = U.b;
    if (w == 0) {
        DrawInfo d;
        d.kind = kNoDraw;
        auto got = [&] { return read_record(P, b, lane, d); };
        bool ok = spin_until(got, P.wait);
        if (!ok) {
            // flagged; the record is still awaited (drained) and, if it
            // comes, drawn as usual, so the sequence's outputs stay whole
            if (lane == 0) cst(P.err, 1u);
            ok = spin_until(got, kWaitTicks);
        }
        if (lane == 0) {
            s_ok = ok ? 1 : 0;
            s_d = d;
        }
    }
    __syncthreads();
    if (!s_ok) {  // the record never came, even after the drain: report the sequence invalid
        if (U.r == 0 && w == 0) write_outputs(P, b, 0, true, 0, lane);
        return;
    }
    const DrawInfo d = s_d;
    if (d.kind != kNoDraw) claim_pieces<DT, VEC>(P, b, d);
}

// A statistics block. Wavefront 0 first reads the decision words of the
// sequence's earlier positions: if the sequence already stopped, the block
// loads none of its rows, counts itself in and (T > 0) spends itself on the
// sequence's draw instead. Otherwise each wavefront streams its chunk range,
// the block's last wavefront writes the block's pieces and counts the block
// in, and the unit's last block decides.
template <int DT, bool VEC, int MODE, bool NT = true>
__device__ inline void stats_block(const Params& P, const Role& U) {
    __shared__ BlockPieces bp;
    __shared__ int32_t s_stop;
    __shared__ DrawInfo s_d;
    const int lane = static_cast<int>(threadIdx.x & (kWave - 1));
    const int w = static_cast<int>(__builtin_amdgcn_readfirstlane(threadIdx.x / kWave));
    if (threadIdx.x == 0) {
        bp.done = 0u;
        s_stop = 0;
    }
    if constexpr (MODE != kRows) {
        if (P.skip && U.i > 0) {
            __syncthreads();
            if (w == 0) {
                const bool stop = sequence_state(P, U.b, U.i, lane) == kStopped;
                DrawInfo d;
                d.kind = kNoDraw;
                if (MODE == kSample && stop && !read_record(P, U.b, lane, d)) d.kind = kNoDraw;
                if (lane == 0) {
                    s_stop = stop ? 1 : 0;
                    s_d = d;
                }
            }
        }
    }
    __syncthreads();
    uint32_t* cnt = P.cnt + static_cast<int64_t>(U.unit) * P.cstride;
    if (s_stop) {
        // counted in; the unit decides nothing (the sequence stopped earlier)
        if (threadIdx.x == 0) {
            const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old + 1u == static_cast<uint32_t>(U.nb)) cst(cnt, 0u);
        }
        if constexpr (MODE == kSample) {
            const DrawInfo d = s_d;
            if (d.kind != kNoDraw) claim_pieces<DT, VEC>(P, U.b, d);
        }
        return;
    }
    const int nwb = min(kWavesPerBlock, U.nw - U.r * kWavesPerBlock);  // wavefronts with work
    if (w >= nwb) return;
    // T > 0: the unit's first wavefront also fetches the draft token's two
    // logits for the decision (off the decider's path)
    const bool fetch = MODE == kSample && U.rows == 2 && U.r == 0 && w == 0;
    int32_t x = -1;
    if (fetch && lane == 0) x = P.tokens[static_cast<int64_t>(U.b) * P.gamma + U.i];
    const int n = stats_wave<DT, VEC, MODE, false, NT>(P, U, U.r * kWavesPerBlock + w, lane, bp.p[w]);
    if (fetch) {
        if (lane == 0) {
            const bool ok = x >= 0 && x < P.V;
            const float lt = ok ? load_one<DT>(unit_row<DT, MODE>(P, U, 0), x) : 0.0f;
            const float ld = ok ? load_one<DT>(unit_row<DT, MODE>(P, U, 1), x) : 0.0f;
            cst(P.tok_l + static_cast<int64_t>(U.unit) * 2, lt);
            cst(P.tok_l + static_cast<int64_t>(U.unit) * 2 + 1, ld);
        }
        complete_before();  // visible before the block counts in
    }
    if (lane == 0) bp.n[w] = n;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(&bp.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    old = __shfl(old, 0, kWave);
    if (old + 1u != static_cast<uint32_t>(nwb)) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    write_pieces<MODE>(P, bp, nwb, lane);
    if (!arrive_last(cnt, static_cast<uint32_t>(U.nb), lane)) return;
    if constexpr (MODE == kSample) decide_sample<DT>(P, U, lane);
    else if constexpr (MODE == kGreedy) decide_greedy(P, U, lane);
    else finish_rows(P, U, lane);
}

// ==========================================================================
// Group-major schedule (T > 0): a group is one sequence's 2*gamma+1 rows (the
// statistics blocks stream 2*gamma of them when the bonus row is deferred);
// its residual blocks (placed kLag groups later in the grid, or at its end)
// fold the group's partials, repeat the accept step for all gamma positions,
// sum the residual of row k (or, deferred, the bonus row's masses) over
// 1024-element subsegments and draw.
// ==========================================================================
// Folding a group's partials (the same exact ldexp combination as above).
struct RowStat {
    float m;
    int32_t arg;
    double s;
};


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
    static_assert(NT == kBlock, "one block folds a group");
    auto sync = [] { __syncthreads(); };
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

// 2^d for the small exponents below (the rounding error of fl(m*c), |d| at
// most 2^-24 |m*c|): the series of e^(d ln 2) to the fifth power, whose
// remainder is below fp64 precision for |d| <= 2^-10; larger d take exp2.
__device__ inline double exp2_small(double d) {
    if (!(fabs(d) <= 0x1.0p-10)) return exp2(d);
    const double x = d * 0.69314718055994530942;
    return 1.0 + x * (1.0 + x * (0.5 + x * (1.0 / 6.0 + x * (1.0 / 24.0 + x * (1.0 / 120.0)))));
}

// The residual constants of a row pair from its folded stats (max m, sum S).
__device__ inline SeqInfo seq_info(int k, bool has_q, float mp, double sp, float mq, double sq, float c32) {
    SeqInfo si;
    const double c = static_cast<double>(c32);
    si.k = k;
    si.has_q = has_q ? 1 : 0;
    si.mcp = mp * c32;
    si.scale_p = exp2_small(static_cast<double>(si.mcp) - static_cast<double>(mp) * c) / sp;
    si.mcq = has_q ? mq * c32 : 0.0f;
    si.rho = has_q ? exp2_small((static_cast<double>(si.mcq) - static_cast<double>(mq) * c) -
                                (static_cast<double>(si.mcp) - static_cast<double>(mp) * c)) * (sp / sq)
                   : 0.0;
    return si;
}

// --------------------------------------------------------------------------
// The accept step, by one wavefront after the group's rows are folded into rs
// (target rows 0..gamma, then draft rows at T > 0): lane i takes draft token
// i, forms alpha in fp64 (greedy: compares the token with the row's argmax),
// compares it with its Philox uniform u (drawn by the caller), and a ballot
// finds the first rejection k. With
// `emit` it writes k, the accepted tokens and the -1 padding (greedy also the
// emitted argmax; the sampled token at k is left to the draw) and the debug
// values. Returns the sequence record the residual needs.
// --------------------------------------------------------------------------
template <bool GREEDY>
__device__ inline SeqInfo accept_wave(const Params& P, uint32_t g, const RowStat* rs, int32_t x, float lt, float ld,
                                      double u, bool emit, bool info = true) {
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
            // (a deferred bonus row is not folded here: its usability is
            // found by the closing blocks that read it)
            ut = (P.defer && i == gamma) || usable(mt, st);
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
                const double ep = (static_cast<double>(lt) - static_cast<double>(mt)) * c;
                const double eq = (static_cast<double>(ld) - static_cast<double>(md)) * c;
                status = accept_test(u, ep, st, eq, sd) ? kAcc : kRej;
                if (emit && (P.dbg_p || P.dbg_q)) {
                    p = exp2(ep) / st;
                    q = exp2(eq) / sd;
                }
            }
            if (emit && P.dbg_p) P.dbg_p[b * gamma + i] = p;
            if (emit && P.dbg_q) P.dbg_q[b * gamma + i] = q;
        }
    }
    SeqInfo mine{};
    if constexpr (!GREEDY) {
        if (info && i <= gamma) mine = seq_info(i, i < gamma, mt, st, md, sd, P.c32);
    }
    const uint64_t stop = __ballot(i < gamma && status != kAcc);
    const int f = stop ? __ffsll(static_cast<unsigned long long>(stop)) - 1 : gamma;
    const int fstat = __shfl(status, f, kWave);
    const bool bonus_ok = __shfl(ut ? 1 : 0, gamma, kWave) != 0;
    const bool invalid = f < gamma ? (fstat == kBad) : !bonus_ok;
    const int k = invalid ? -1 : f;
    // (all gamma accepted with the bonus row deferred: the outputs are written
    // with the bonus draw, once the row is known to be usable)
    const bool later = !GREEDY && P.defer && k == gamma;
    if (emit && !later) {
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
    rr.prow = group_row<DT>(P, g, static_cast<uint32_t>(s.k));
    rr.qrow = s.has_q ? group_row<DT>(P, g, static_cast<uint32_t>(P.gamma + 1 + s.k)) : nullptr;
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
// The same two steps on up to kDrawTiles*64 masses held in registers (one
// load round trip); the totals and prefix sums are formed exactly as above.
constexpr int kDrawTiles = 4;

// Tiles from nt on (wave-uniform) hold only zeros: their scans are skipped,
// which leaves every result as it would be.
template <int NT = kDrawTiles>
__device__ inline double regs_scan(const double* v, double* incl, int lane, int nt = NT) {
    double base = 0.0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t < nt) {
            incl[t] = base + wave_scan_incl(v[t]);
            base = lane_f64(incl[t], kWave - 1);
        } else {
            incl[t] = base;
        }
    }
    return base;
}

template <int NT = kDrawTiles>
__device__ inline int32_t regs_find(const double* v, const double* incl, double t, int lane, double& before,
                                    int nt = NT) {
    int32_t last = -1;
    double last_before = 0.0;
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        if (k >= nt) break;
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
__device__ inline void draw(const Params& P, uint32_t g, const SeqInfo& in, int lane, double ud, bool dead) {
    const int32_t nsub = P.nsub;
    double* sr = P.sub_r + static_cast<int64_t>(g) * nsub;
    const double u = __shfl(ud, in.k, kWave);  // lane i holds the draw's uniform for k = i
    double Z, target, before = 0.0;
    int32_t sel;
    bool from_p = false;  // no residual mass left by rounding: draw from p_k
    if (nsub <= kDrawTiles * kWave) {
        double v[kDrawTiles], incl[kDrawTiles];
#pragma unroll
        for (int t = 0; t < kDrawTiles; ++t) v[t] = t * kWave + lane < nsub ? cld(sr + t * kWave + lane) : 0.0;
        const int nt = static_cast<int>((nsub + kWave - 1) / kWave);
        Z = regs_scan(v, incl, lane, nt);
        from_p = !(Z > 0.0);
        if (from_p) {
            p_masses<DT, VEC>(P, g, in, sr, lane);
#pragma unroll
            for (int t = 0; t < kDrawTiles; ++t) v[t] = t * kWave + lane < nsub ? cld(sr + t * kWave + lane) : 0.0;
            target = u * regs_scan(v, incl, lane, nt);
        } else {
            target = u * Z;
        }
        sel = regs_find(v, incl, target, lane, before, nt);
    } else {
        Z = scan_total(sr, nsub, lane);
        from_p = !(Z > 0.0);
        if (from_p) p_masses<DT, VEC>(P, g, in, sr, lane);
        target = u * (from_p ? scan_total(sr, nsub, lane) : Z);
        sel = scan_find(sr, nsub, target, lane, before);
    }
    if (dead) return;  // (the caller writes the whole row as invalid)
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
    const double incl = before + wave_scan_incl(local);
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
// Deferred bonus row (group-major, T > 0, no per-row debug output): the
// statistics blocks do not stream target row gamma, which only a sequence
// that accepts all gamma draft tokens needs; that sequence's closing blocks
// read it instead of a residual row. A subsegment's mass is formed at its own
// integer reference R_s = ceil(max_s * c) from its maximum: the sum of
// 2^(fl(x*c - R_s)) (fp32 per element, fp64 in element order per lane, then
// across the wavefront), stored with R_s. The draw rebases the masses to the
// largest reference by exact powers of two, so the draw from p (its
// normalisation cancels) needs neither the row's maximum nor its sum first. A
// NaN or +inf logit, or one whose x*c overflows, marks its subsegment (mass
// NaN): the row is then unusable and the sequence reported invalid, as when
// the bonus row is folded with the others.
// --------------------------------------------------------------------------
template <int DT, bool VEC>
__device__ inline void bonus_masses(const Params& P, uint32_t g, int32_t i0, int32_t stride, int lane) {
    const float c = P.c32;
    ResidRow rr{};
    rr.prow = group_row<DT>(P, g, static_cast<uint32_t>(P.gamma));
    rr.qrow = nullptr;
    double* sr = P.sub_r + static_cast<int64_t>(g) * P.nsub;
    float* sR = P.sub_R + static_cast<int64_t>(g) * P.nsub;
    for (int32_t i = i0; i < P.nsub; i += stride) {
        float x[16], none[16];
        load_sub<DT, VEC>(rr, false, static_cast<int64_t>(i) * kSub + 16 * lane, P.V, x, none);
        float mx = -INFINITY;
        bool bad = false;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            bad |= !(x[v] == x[v]) || x[v] == INFINITY;
            mx = fmaxf(mx, x[v]);
        }
        mx = wave_max(mx);
        bad = __ballot(bad) != 0;
        float R = kRUnset;
        if (mx * c > kRUnset + 1.0f) {
            const float Rn = ceilf(mx * c);
            if (Rn < 3.0e38f) R = Rn;
            else bad = true;
        }
        double t = 0.0;
        if (R > kRUnset) {
#pragma unroll
            for (int v = 0; v < 16; ++v) t += static_cast<double>(__builtin_amdgcn_exp2f(fmaf(x[v], c, -R)));
        }
        t = wave_sum(t);
        if (lane == 0) {
            cst(sr + i, bad ? static_cast<double>(NAN) : t);
            cst(sR + i, R);
        }
    }
}

// The deferred bonus draw and the sequence's outputs (the group's last
// closing wavefront, every closing block counted in): x is lane's draft
// token (lane < gamma). The masses, rebased to the largest reference, are
// scanned as in draw(); the chosen subsegment is read again and its elements'
// masses formed exactly as in bonus_masses, scaled by the same power of two.
template <int DT, bool VEC>
__device__ inline void draw_bonus(const Params& P, uint32_t g, int32_t x, int lane, double ud, bool dead) {
    const int32_t gamma = P.gamma, nsub = P.nsub, nt = gamma + 1;
    const float c = P.c32;
    const double* sr = P.sub_r + static_cast<int64_t>(g) * nsub;
    const float* sR = P.sub_R + static_cast<int64_t>(g) * nsub;
    const double u = __shfl(ud, gamma, kWave);  // lane i holds the draw's uniform for k = i
    float R = kRUnset;
    bool bad = false;
    for (int32_t i = lane; i < nsub; i += kWave) {
        const double m = cld(sr + i);
        bad |= !(m == m);
        R = fmaxf(R, cld(sR + i));
    }
    R = wave_max(R);
    bad = __ballot(bad) != 0;
    auto val = [&](int32_t i) {
        if (i >= nsub) return 0.0;
        const float r = cld(sR + i);
        return r > kRUnset ? ldexp(cld(sr + i), static_cast<int>(fmaxf(r - R, -1100.0f))) : 0.0;
    };
    double Z = 0.0, target = 0.0, before = 0.0;
    int32_t sel = -1;
    if (!bad) {
        if (nsub <= kDrawTiles * kWave) {
            double v[kDrawTiles], incl[kDrawTiles];
#pragma unroll
            for (int t = 0; t < kDrawTiles; ++t) v[t] = val(t * kWave + lane);
            const int nt = static_cast<int>((nsub + kWave - 1) / kWave);
            Z = regs_scan(v, incl, lane, nt);
            if (Z > 0.0) {
                target = u * Z;
                sel = regs_find(v, incl, target, lane, before, nt);
            }
        } else {  // many subsegments: tiles of 64 in order, the total first, then the crossing
            for (int32_t t0 = 0; t0 < nsub; t0 += kWave) Z += lane_f64(wave_scan_incl(val(t0 + lane)), kWave - 1);
            if (Z > 0.0) {
                target = u * Z;
                double base = 0.0, last_before = 0.0;
                int32_t last = -1;
                for (int32_t t0 = 0; t0 < nsub && sel < 0; t0 += kWave) {
                    const double v = val(t0 + lane);
                    const double incl = base + wave_scan_incl(v);
                    const double prev = lane_before(incl);
                    const double excl = lane == 0 ? base : prev;
                    const uint64_t hit = __ballot(v > 0.0 && excl <= target && target < incl);
                    if (hit) {
                        const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
                        sel = t0 + l;
                        before = __shfl(excl, l, kWave);
                    } else {
                        const uint64_t any = __ballot(v > 0.0);
                        if (any) {
                            const int l = 63 - __clzll(static_cast<unsigned long long>(any));
                            last = t0 + l;
                            last_before = __shfl(excl, l, kWave);
                        }
                    }
                    base = lane_f64(incl, kWave - 1);
                }
                if (sel < 0) {
                    sel = last;
                    before = last_before;
                }
            }
        }
    }
    if (dead) return;  // (the caller writes the whole row as invalid)
    const bool ok = !bad && Z > 0.0 && sel >= 0;
    int32_t pick = -1;
    if (ok) {
        const float Rs = cld(sR + sel);
        const double sc = ldexp(1.0, static_cast<int>(fmaxf(Rs - R, -1100.0f)));
        ResidRow rr{};
        rr.prow = group_row<DT>(P, g, static_cast<uint32_t>(gamma));
        rr.qrow = nullptr;
        const int64_t j0 = static_cast<int64_t>(sel) * kSub + 16 * lane;
        float xs[16], none[16];
        load_sub<DT, VEC>(rr, false, j0, P.V, xs, none);
        double mv[16];
        double local = 0.0;
        int32_t mylast = -1;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            mv[v] = static_cast<double>(__builtin_amdgcn_exp2f(fmaf(xs[v], c, -Rs))) * sc;
            local += mv[v];
            if (mv[v] > 0.0) mylast = static_cast<int32_t>(j0 + v);
        }
        const double incl = before + wave_scan_incl(local);
        const double prev = lane_before(incl);
        const double excl = lane == 0 ? before : prev;
        const uint64_t hit = __ballot(local > 0.0 && excl <= target && target < incl);
        if (hit) {
            const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
            int32_t p = -1;
            if (lane == l) {
                double run = excl;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    run += mv[v];
                    if (p < 0 && mv[v] > 0.0 && run > target) p = static_cast<int32_t>(j0 + v);
                }
                if (p < 0) p = mylast;
            }
            pick = __shfl(p, l, kWave);
        } else {  // rounding: the last element with mass in the subsegment
            const uint64_t mass = __ballot(mylast >= 0);
            const int l = mass ? 63 - __clzll(static_cast<unsigned long long>(mass)) : 0;
            pick = __shfl(mylast, l, kWave);
        }
    }
    int32_t* out = P.out_tokens + static_cast<int64_t>(g) * nt;
    if (lane < gamma) cst(out + lane, ok ? x : -1);
    if (lane == gamma) cst(out + gamma, ok ? pick : -1);
    if (lane == 0) cst(P.out_n + g, ok ? gamma : -1);
}

// --------------------------------------------------------------------------
// Group finishers and the residual block
// --------------------------------------------------------------------------
// Waits (one lane) until every statistics block of group g has counted in.
// Returns 0 if they did within the bound; 1 if the bound ran out (the sticky
// error word is then set) but they did within the drain that follows; 2 if
// not even then.
// (phase 2: the second phase's count, the word after the first's)
__device__ inline int wait_published(const Params& P, uint32_t g, int phase = 0) {
    const uint32_t* cnt = P.cnt_s + static_cast<int64_t>(g) * kSyncStride + (phase == 2 ? 1 : 0);
    const uint32_t want = static_cast<uint32_t>(phase == 2 ? P.psb2 : P.sb);
    if (spin_count(cnt, want, P.wait)) return 0;
    cst(P.err, 1u);
    return spin_count(cnt, want, kWaitTicks) ? 1 : 2;
}

// Two phases: group g's decision record, kGroupRecWords 64-bit words after
// the groups' void words, each carrying this call's epoch in its high half
// (a reader that sees the epoch in all of them has the whole record): the
// status (kind << 8 | k), then fl(max*c) of target and draft row k, rho and
// scale_p (each fp64 as two halves). Written once per call by the group's
// decider; nothing needs clearing between calls.
constexpr int kGroupRecWords = 8;
enum : uint32_t { kRecStop = 1, kRecCont = 2, kRecVoid = 3 };
__device__ inline uint64_t* group_rec(const Params& P, uint32_t g) {
    return P.dec + P.B + static_cast<int64_t>(g) * kGroupRecWords;
}
struct GroupRec {
    uint32_t kind;
    int32_t k;
    float mcp, mcq;
    double rho, scale_p;
};
// One read of the record (one wavefront): false until every word is current.
__device__ inline bool read_group_rec(const Params& P, uint32_t g, int lane, GroupRec& r) {
    const uint64_t* w = group_rec(P, g);
    const uint64_t v = lane < 7 ? cld64(w + lane) : (static_cast<uint64_t>(P.epoch) << 32);
    if (__ballot(static_cast<uint32_t>(v >> 32) != P.epoch) != 0) return false;
    const uint32_t x = static_cast<uint32_t>(v);
    const uint32_t w0 = __shfl(x, 0, kWave);
    r.kind = w0 >> 8;
    r.k = static_cast<int32_t>(w0 & 0xFFu);
    r.mcp = __uint_as_float(__shfl(x, 1, kWave));
    r.mcq = __uint_as_float(__shfl(x, 2, kWave));
    r.rho = __hiloint2double(static_cast<int>(__shfl(x, 4, kWave)), static_cast<int>(__shfl(x, 3, kWave)));
    r.scale_p = __hiloint2double(static_cast<int>(__shfl(x, 6, kWave)), static_cast<int>(__shfl(x, 5, kWave)));
    return true;
}
// Group-major: the word that marks group g's outputs void in this call (a wait
// of one of its closing blocks ran out); the group's last closing block then
// writes the whole row as invalid.
__device__ inline uint64_t* void_word(const Params& P, uint32_t g) { return P.dec + g; }

// Two phases, T > 0: the decider of group g (one block, after every group's
// first-phase statistics blocks). Once the first phase's rows have counted
// in, it folds them and takes the accept step for positions 0..p0-1 exactly
// as the residual blocks do for all positions. A rejection or an unusable row
// there ends the sequence: the decider writes a record with k and row k's
// residual constants; the second phase's statistics blocks of the group then
// load nothing, and its residual blocks skip the fold (the first of them
// writes the outputs, the draw the token at k). All p0 accepted: the record
// says so, and the residual blocks fold the whole group as in one phase. A
// wait that runs out makes the record void (the outputs -1). The decider
// writes nothing else, so the record leaves as soon as it is known, and
// resets the first phase's count.
template <int DT, bool VEC>
__device__ inline void decide_block(const Params& P, uint32_t g, char* dyn) {
    __shared__ RowStat rs[2 * SPEC_MAX_GAMMA + 1];
    __shared__ int s_st;
    const int lane = static_cast<int>(threadIdx.x & (kWave - 1));
    const int w = static_cast<int>(threadIdx.x / kWave);
    const int32_t gamma = P.gamma, p0 = P.p0, nt = gamma + 1;
    int32_t x = 0;
    float lt = 0.0f, ld = 0.0f;
    double u = 0.0;
    if (w == 0 && lane < p0) {
        u = philox_uniform(P.seed, static_cast<uint32_t>(g + P.b_offset), static_cast<uint32_t>(lane), 0u);
        x = P.tokens[static_cast<int64_t>(g) * gamma + lane];
        if (x >= 0 && x < P.V) {
            lt = load_one<DT>(group_row<DT>(P, g, static_cast<uint32_t>(lane)), x);
            ld = load_one<DT>(group_row<DT>(P, g, static_cast<uint32_t>(nt + lane)), x);
        }
    }
    uint32_t* cnt = P.cnt_s + static_cast<int64_t>(g) * kSyncStride;
    if (threadIdx.x == 0) {
        int st = 0;
        if (!spin_count(cnt, static_cast<uint32_t>(P.sb), P.wait)) {
            cst(P.err, 1u);
            st = spin_count(cnt, static_cast<uint32_t>(P.sb), kWaitTicks) ? 1 : 2;
        }
        s_st = st;
    }
    __syncthreads();
    after_complete();
    if (s_st == 0) merge_group<false, kBlock>(P, g, dyn, rs);  // (the second phase's rows are not used)
    if (w != 0) return;
    const int i = lane;
    uint32_t kind = kRecVoid;
    int32_t k = -1;
    double rho = 0.0, scale_p = 0.0;
    float mcp = 0.0f, mcq = 0.0f;
    if (s_st == 0) {
        int status = kAcc;
        float mt = NAN, md = NAN;
        double st = NAN, sd = NAN;
        if (i < p0) {
            mt = rs[i].m;
            st = rs[i].s;
            md = rs[nt + i].m;
            sd = rs[nt + i].s;
            if (!usable(mt, st) || !usable(md, sd) || !(x >= 0 && x < P.V)) {
                status = kBad;
            } else {
                const double c = static_cast<double>(P.c32);
                const double ep = (static_cast<double>(lt) - static_cast<double>(mt)) * c;
                const double eq = (static_cast<double>(ld) - static_cast<double>(md)) * c;
                status = accept_test(u, ep, st, eq, sd) ? kAcc : kRej;
            }
        }
        const uint64_t stop = __ballot(i < p0 && status != kAcc);
        if (stop) {
            const int f = __ffsll(static_cast<unsigned long long>(stop)) - 1;
            const bool invalid = __shfl(status, f, kWave) == kBad;
            k = invalid ? -1 : f;
            kind = invalid ? kRecVoid : kRecStop;
            if (!invalid) {
                SeqInfo mine{};
                if (i == f) mine = seq_info(i, true, mt, st, md, sd, P.c32);
                mcp = __shfl(mine.mcp, f, kWave);
                mcq = __shfl(mine.mcq, f, kWave);
                rho = __shfl(mine.rho, f, kWave);
                scale_p = __shfl(mine.scale_p, f, kWave);
            }
        } else {
            kind = kRecCont;
        }
    }
    uint64_t* r = group_rec(P, g);
    const uint64_t rb = __double_as_longlong(rho), sb = __double_as_longlong(scale_p);
    uint32_t v = 0u;
    if (i == 0) v = (kind << 8) | static_cast<uint32_t>(k < 0 ? 0 : k);
    if (i == 1) v = __float_as_uint(mcp);
    if (i == 2) v = __float_as_uint(mcq);
    if (i == 3) v = static_cast<uint32_t>(rb);
    if (i == 4) v = static_cast<uint32_t>(rb >> 32);
    if (i == 5) v = static_cast<uint32_t>(sb);
    if (i == 6) v = static_cast<uint32_t>(sb >> 32);
    if (i < 7) cst64(r + i, tagged(P, v));
    // every first-phase block has counted in (unless even the drain ran out:
    // then the count is left for the status call's scrub)
    if (i == 0 && s_st != 2) cst(cnt, 0u);
}

// T > 0: one residual block of group g (idx in [0, rb)). Once every
// statistics block of g has counted in, the block folds g's partials and
// repeats the accept step (block 0 writes the results); then wavefront w takes
// subsegments idx*4 + w + t*rb*4, t < subs_per_wave(), loading all of them
// before summing. The group's last residual block draws the token and resets
// the group's counters for the next call.
template <int DT, bool VEC>
__device__ inline void group_resid_block(const Params& P, uint32_t g, uint32_t idx, char* dyn) {
    __shared__ RowStat rs[2 * SPEC_MAX_GAMMA + 1];
    __shared__ SeqInfo shi;
    __shared__ SeqInfo s_info[SPEC_MAX_GAMMA + 1];
    __shared__ int s_st;
    __shared__ uint32_t s_last;
    const int lane = static_cast<int>(threadIdx.x & (kWave - 1));
    const int w = static_cast<int>(threadIdx.x / kWave);
    const int32_t gamma = P.gamma;
    // the draft tokens, their two logits, the accept uniforms and the draw's
    // uniform for every possible k do not depend on the statistics: they are
    // loaded and drawn before the wait
    int32_t x = 0;
    float lt = 0.0f, ld = 0.0f;
    double u = 0.0;   // the accept uniform of position lane
    double ud = 0.0;  // the draw's uniform if k = lane
    if (w == 0 && lane <= gamma)
        ud = philox_uniform(P.seed, static_cast<uint32_t>(g + P.b_offset), static_cast<uint32_t>(lane), 1u);
    if (w == 0 && lane < gamma) {
        u = philox_uniform(P.seed, static_cast<uint32_t>(g + P.b_offset), static_cast<uint32_t>(lane), 0u);
        x = P.tokens[static_cast<int64_t>(g) * gamma + lane];
        if (x >= 0 && x < P.V) {
            lt = load_one<DT>(group_row<DT>(P, g, static_cast<uint32_t>(lane)), x);
            ld = load_one<DT>(group_row<DT>(P, g, static_cast<uint32_t>(gamma + 1 + lane)), x);
        }
    }
    // two phases: the decider's record first. A sequence that stopped within
    // the first phase takes k and its constants from it; one that did not
    // waits for the second phase's statistics and folds the group below.
    __shared__ GroupRec s_rec;
    bool fold = true;
    if (P.p0 > 0) {
        if (w == 0) {
            GroupRec r;
            auto got = [&] { return read_group_rec(P, g, lane, r); };
            if (!spin_until(got, P.wait)) {  // flagged, and the group's outputs void
                if (lane == 0) {
                    cst(P.err, 1u);
                    cst64(void_word(P, g), tagged(P, 1u));
                }
                r.kind = kRecVoid;
            }
            if (lane == 0) s_rec = r;
        }
        __syncthreads();
        fold = s_rec.kind == kRecCont;
    }
    if (fold && threadIdx.x == 0) {
        const int st = wait_published(P, g, P.p0 > 0 ? 2 : 0);
        if (st != 0) cst64(void_word(P, g), tagged(P, 1u));  // the wait ran out: the group's outputs are void
        s_st = st;
    }
    __syncthreads();
    after_complete();
    SeqInfo in;
    in.k = -1;
    if (!fold && s_rec.kind == kRecStop) {
        const GroupRec r = s_rec;
        in.k = r.k;
        in.has_q = 1;
        in.mcp = r.mcp;
        in.mcq = r.mcq;
        in.rho = r.rho;
        in.scale_p = r.scale_p;
    }
    if (!fold && idx == 0 && w == 0) {  // stopped (or void) within the first phase: k, the accepted tokens, -1 after k
        const int32_t k = in.k;
        if (lane <= gamma && (k < 0 || lane != k))
            cst(P.out_tokens + static_cast<int64_t>(g) * (gamma + 1) + lane, lane < k ? x : -1);
        if (lane == 0) cst(P.out_n + g, k);
    }
    if (fold && s_st == 0) {
        merge_group<false, kBlock>(P, g, dyn, rs);
        // wavefront 0 takes the accept step while wavefront 1 forms the
        // residual constants of every row pair (the accept step's ballot
        // picks one)
        if (w == 0) {
            const SeqInfo si = accept_wave<false>(P, g, rs, x, lt, ld, u, idx == 0, false);
            if (lane == 0) shi = si;
        } else if (w == 1 && lane <= gamma) {
            s_info[lane] = seq_info(lane, lane < gamma, rs[lane].m, rs[lane].s, lane < gamma ? rs[gamma + 1 + lane].m : 0.0f,
                                    lane < gamma ? rs[gamma + 1 + lane].s : 0.0, P.c32);
        }
        __syncthreads();
        in = shi;
        if (in.k >= 0) in = s_info[in.k];
    }
    if (in.k >= 0 && P.defer && in.k == gamma) {
        bonus_masses<DT, VEC>(P, g, static_cast<int32_t>(idx) * kWavesPerBlock + w, P.rb * kWavesPerBlock, lane);
    } else if (in.k >= 0) {
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
                if (t < P.spw && i < P.nsub) raw[t].load(rr, has_q, static_cast<int64_t>(i) * kSub + 16 * lane, P.V);
            }
#pragma unroll
            for (int t = 0; t < NS; ++t) {
                const int32_t i = i0 + t * stride;
                if (t >= P.spw || i >= P.nsub) break;
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
    // every residual block of g has counted in. The void word and the counts
    // this block resets are loaded beside the draw's first loads: only the
    // draw's writes wait for the word, and the resets follow the draw.
    uint32_t* cnt_s = P.cnt_s + static_cast<int64_t>(g) * kSyncStride;
    const uint64_t vw = cld64(void_word(P, g));
    uint32_t c1 = 0, c2 = 0;
    if (lane == 0) {
        c1 = cld(cnt_s);
        if (P.p0 > 0) c2 = cld(cnt_s + 1);
    }
    const bool dead = static_cast<uint32_t>(vw >> 32) == P.epoch;
    if (in.k >= 0 && P.defer && in.k == gamma) {
        draw_bonus<DT, VEC>(P, g, x, lane, ud, dead);
    } else if (in.k >= 0) {
        draw<DT, VEC>(P, g, in, lane, ud, dead);
    }
    if (dead) {  // a closing block's wait ran out: the whole row is reported invalid
        if (lane <= gamma) cst(P.out_tokens + static_cast<int64_t>(g) * (gamma + 1) + lane, -1);
        if (lane == 0) {
            cst(P.out_n + g, -1);
            if (P.dbg_z) P.dbg_z[g] = NAN;
        }
    }
    if (lane == 0) {
        // the statistics count, once complete (unless even a drain ran out:
        // then it is left for the status call's scrub; in two phases the
        // decider has reset it)
        if (c1 == static_cast<uint32_t>(P.sb)) cst(cnt_s, 0u);
        cst(cnt_r, 0u);
        if (dead) cst64(void_word(P, g), 0ull);  // (a mark never outlives its call)
        // two phases: the second phase's count, once all its blocks have
        // counted in (those of a stopped sequence load nothing and come soon)
        if (P.p0 > 0) {
            uint32_t* cnt2 = cnt_s + 1;
            if (c2 == static_cast<uint32_t>(P.psb2) || spin_count(cnt2, static_cast<uint32_t>(P.psb2), kWaitTicks))
                cst(cnt2, 0u);
        }
    }
}

// T == 0: the one closing block of group g (the sequence's gamma + 1 target
// rows). Once every statistics block of g has counted in, it folds the rows'
// argmax partials and takes the greedy step (accept while the draft token is
// the row's argmax, emit the argmax at the first mismatch or the bonus row),
// then resets the group's count for the next call.
__device__ inline void group_greedy_block(const Params& P, uint32_t g, char* dyn) {
    __shared__ RowStat rs[2 * SPEC_MAX_GAMMA + 1];
    __shared__ int s_st;
    const int lane = static_cast<int>(threadIdx.x & (kWave - 1));
    const int w = static_cast<int>(threadIdx.x / kWave);
    const int32_t gamma = P.gamma;
    int32_t x = 0;  // the draft tokens do not depend on the statistics: loaded before the wait
    if (w == 0 && lane < gamma) x = P.tokens[static_cast<int64_t>(g) * gamma + lane];
    if (threadIdx.x == 0) s_st = wait_published(P, g);
    __syncthreads();
    after_complete();
    if (s_st == 0) {
        merge_group<true, kBlock>(P, g, dyn, rs);
        if (w == 0) (void)accept_wave<true>(P, g, rs, x, 0.0f, 0.0f, 0.0, true);
    } else if (w == 0) {  // the wait ran out: the sequence is reported invalid
        if (lane <= gamma) cst(P.out_tokens + static_cast<int64_t>(g) * (gamma + 1) + lane, -1);
        if (lane == 0) cst(P.out_n + g, -1);
    }
    // every statistics block has counted in (unless even the drain ran out:
    // then the count is left for the status call's scrub)
    if (w == 0 && lane == 0 && s_st != 2) cst(P.cnt_s + static_cast<int64_t>(g) * kSyncStride, 0u);
}

// The group-major kernel: statistics blocks stream whole groups; at T > 0 the
// group's residual blocks take the accept step and the draw, at T == 0 one
// block per group takes the greedy step.
template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kBlock) void k_group(Params P) {
    extern __shared__ __align__(16) char dyn[];
    int kind;
    uint32_t g, idx;
    int phase;
    decode_block(P, blockIdx.x, kind, g, idx, phase);
    const int lane = static_cast<int>(threadIdx.x & (kWave - 1));
    if (kind == kStatsBlock) {
        __shared__ BlockPieces bp;
        const int w = static_cast<int>(__builtin_amdgcn_readfirstlane(threadIdx.x / kWave));
        const int pnw = phase == 2 ? P.pnw2 : P.nw;
        const int nwb = min(kWavesPerBlock, pnw - static_cast<int>(idx) * kWavesPerBlock);  // wavefronts with work
        if (threadIdx.x == 0) {
            bp.done = 0u;
            bp.skip = 0u;
            if (phase == 2) {  // the sequence stopped within the first phase: nothing to load
                uint64_t w0 = 0;
                auto known = [&] {
                    w0 = cld64(group_rec(P, g));
                    return static_cast<uint32_t>(w0 >> 32) == P.epoch;
                };
                // (the decider precedes every second-phase block in the grid;
                // a wait that runs out loads the rows, which is never wrong)
                const bool k = SPECVERIFY_PHASE2_WAIT ? spin_until(known, P.wait) : known();
                bp.skip = k && (static_cast<uint32_t>(w0) >> 8) != kRecCont;
            }
        }
        __syncthreads();
        if (w >= nwb) return;
        Role U;
        U.kind = kStatsBlock;
        U.unit = g;
        U.i = phase;
        U.b = static_cast<int32_t>(g);
        U.r = static_cast<int32_t>(idx);
        U.rows = phase == 1 ? 2 * P.p0 : (phase == 2 ? 2 * (P.gamma - P.p0) : P.srows);
        U.nw = pnw;
        U.nb = phase == 2 ? P.psb2 : P.sb;
        int n = 0;
        if (bp.skip) n = 0;
        else if (static_cast<int32_t>(g) >= P.cached_from)  // (the last groups: their rows k are read again soon)
            n = stats_wave<DT, VEC, MODE, true, false>(P, U, idx * kWavesPerBlock + w, lane, bp.p[w]);
        else
            n = stats_wave<DT, VEC, MODE, true>(P, U, idx * kWavesPerBlock + w, lane, bp.p[w]);
        // count this wavefront in at the block; the last one writes the block's pieces
        if (lane == 0) bp.n[w] = n;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        uint32_t old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(&bp.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        old = __shfl(old, 0, kWave);
        if (old + 1u != static_cast<uint32_t>(nwb)) return;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        write_pieces<MODE>(P, bp, nwb, lane);
        // the closing blocks of g watch this count reach sb (psb2: the second phase's, the next word)
        complete_before();
        if (lane == 0)
            (void)__hip_atomic_fetch_add(P.cnt_s + static_cast<int64_t>(g) * kSyncStride + (phase == 2 ? 1 : 0), 1u,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if constexpr (MODE == kGreedy) {
        group_greedy_block(P, g, dyn);
    } else if (kind == kDecideBlock) {
        decide_block<DT, VEC>(P, g, dyn);
    } else {
        group_resid_block<DT, VEC>(P, g, idx, dyn);
    }
}

// --------------------------------------------------------------------------
// The kernel: one launch per call.
// --------------------------------------------------------------------------
template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kBlock) void k_verify(Params P) {
    const Role U = role_of<MODE>(P);
    if constexpr (MODE == kSample) {
        if (U.kind == kResidBlock) {
            resid_block<DT, VEC>(P, U);
            return;
        }
    }
    // (T == 0 with ordinary loads: measured 28.4 against 29.0 us on the greedy
    // workload; at T > 0 non-temporal loads are as fast or faster)
    stats_block<DT, VEC, MODE, MODE != kGreedy>(P, U);
}


// ==========================================================================
// Draft-side sampling ([Ch15] 15.1.2 step 1: each draft token is drawn from
// the draft model's distribution and its probability kept; [CSDN] 2.1, stage 1
// of speculative_decode()). Row (b, t) of a [B, n, V] block of draft logits
// gives x, the smallest j whose ascending cumulative mass of softmax(l/T)
// exceeds u*S, with u the Philox uniform of counter (b + b_offset, pos0 + t,
// DRAFT), and q = p(x); at T == 0, x = the first argmax and q = 1.
//
// Rows are independent, so nothing waits. Wavefront w of a row loads its range
// of kDraftCw chunks in one go and writes one partial: at T > 0 (max, integer
// reference R, sum of 2^(fl(x*c - R)) in fp64 over fp32 groups), at T == 0
// (max, first index of it). The row's last block to count in folds the
// partials, finds the range where the cumulative mass crosses u*S, loads that
// range again (one wavefront, 16 KiB) and finds the element in ascending
// order from the same fp32 element values, scaled to the row's reference by
// an exact power of two.
// ==========================================================================
constexpr int kDraftCw = SPECVERIFY_DRAFT_CW;  // chunks per wavefront range
constexpr int kFinTiles = 2;  // range sums the finishing wavefront holds: 64 * kFinTiles (more: three passes)
constexpr int kDraftStride = 32;    // words between two row counters
constexpr uint32_t kPurposeDraft = 2u;

struct DraftParams {
    const void* logits;  // [rows, V], row r = b * n + t
    int64_t rows;
    int32_t n, V, nchunk;
    int32_t nw;   // wavefront ranges per row
    int32_t nbr;  // blocks per row
    float c32;    // log2(e) / T
    uint64_t seed;
    int64_t pos0, b_offset;
    int32_t* out_tokens;  // [rows]
    double* out_q;        // [rows] or null
    // per range k of row r, kDraftWords 64-bit words at part[(r * nw + k) * kDraftWords],
    // each (epoch << 32 | payload): T > 0 the fp32 sum of 2^(fl(x*c - R)), the
    // integer reference R, the fp32 sum of 2^t * t (t = fl(x*c - R), entropy
    // wanted); T == 0 the maximum and its first index
    uint64_t* part;
    uint32_t epoch;       // this call's tag
    double* out_h;        // [rows] or null: entropy of softmax(l/T) per row
    uint32_t* err;        // sticky error word (a bounded wait ran out)
    uint64_t wait;        // bound on the closing wavefront's wait, in wall-clock ticks
};
constexpr int kDraftWords = 3;
__device__ inline uint64_t tagged(uint32_t epoch, uint32_t payload) {
    return (static_cast<uint64_t>(epoch) << 32) | payload;
}

// The token of range `sel` (chunks c0 .. c0 + kDraftCw - 1 of the row, loaded
// into q): elements visited in ascending index order as tiles (Tiles), each
// lane's tile mass the fp64 sum of 2^(fl(x*c - rs)) * sc (sc = 2^(rs - R), an
// exact rescaling to the row's reference), the first element where the
// cumulative mass, starting at `before`, exceeds `target`; if rounding leaves
// none, the last element with mass. Returns (in every lane) the token and, in
// `mass`, its scaled mass.
template <int DT, bool VEC, int N>
__device__ __attribute__((always_inline)) inline int32_t draft_pick(const typename Chunk<DT, VEC>::Raw* q, int64_t c0, float c, float rs, double sc,
                                     double before, double target, int lane, double& mass) {
    using C = Chunk<DT, VEC>;
    using TL = Tiles<DT, VEC>;
    int32_t last = -1;
    double last_m = 0.0;
    double run = before;
#pragma unroll
    for (int u = 0; u < N; ++u) {
        float x[C::EPL];
        typename C::Raw r = q[u];
        opaque(r);  // expanded here, one chunk at a time
        C::expand(r, x);
#pragma unroll
        for (int t = 0; t < TL::PER_CHUNK; ++t) {
            double lm = 0.0, ml = 0.0;
            int32_t mylast = -1;
#pragma unroll
            for (int e = 0; e < TL::EPT; ++e) {
                const int v = VEC ? e : t;
                const double m = static_cast<double>(__builtin_amdgcn_exp2f(fmaf(x[v], c, -rs))) * sc;
                lm += m;
                if (m > 0.0) {
                    mylast = static_cast<int32_t>(C::index_of(c0 + u, lane, v));
                    ml = m;
                }
            }
            const double incl = run + wave_scan_incl(lm);
            const double prev = lane_before(incl);
            const double excl = lane == 0 ? run : prev;
            const uint64_t hit = __ballot(lm > 0.0 && excl <= target && target < incl);
            if (hit) {
                const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
                int32_t pick = -1;
                double pm = 0.0;
                if (lane == l) {
                    double r2 = excl;
#pragma unroll
                    for (int e = 0; e < TL::EPT; ++e) {
                        const int v = VEC ? e : t;
                        const double m = static_cast<double>(__builtin_amdgcn_exp2f(fmaf(x[v], c, -rs))) * sc;
                        r2 += m;
                        if (pick < 0 && m > 0.0 && r2 > target) {
                            pick = static_cast<int32_t>(C::index_of(c0 + u, lane, v));
                            pm = m;
                        }
                    }
                    if (pick < 0) {
                        pick = mylast;
                        pm = ml;
                    }
                }
                mass = __shfl(pm, l, kWave);
                return __shfl(pick, l, kWave);
            }
            const uint64_t any = __ballot(mylast >= 0);
            if (any) {
                const int l = 63 - __clzll(static_cast<unsigned long long>(any));
                last = __shfl(mylast, l, kWave);
                last_m = __shfl(ml, l, kWave);
            }
            run = lane_f64(incl, kWave - 1);
        }
    }
    mass = last_m;
    return last;
}

// The token of an N-chunk range starting at chunk c0 (loaded into q): the
// chunks' masses first, independently of one another (fp64, tiles in
// ascending order), then the chunk where the cumulative mass, starting at
// `before`, first exceeds `target` (if rounding leaves none, the last chunk
// with mass), then the element in that chunk (draft_pick). -1 if the range
// has no mass.
template <int DT, bool VEC, int N>
__device__ __attribute__((always_inline)) inline int32_t draft_pick_range(const typename Chunk<DT, VEC>::Raw* q, int64_t c0, float c, float rs,
                                           double sc, double before, double target, int lane, double& mass) {
    using C = Chunk<DT, VEC>;
    double cm[N];
#pragma unroll
    for (int u = 0; u < N; ++u) {
        float x[C::EPL];
        typename C::Raw r = q[u];
        opaque(r);
        C::expand(r, x);
        double lm = 0.0;
#pragma unroll
        for (int v = 0; v < C::EPL; ++v) lm += static_cast<double>(__builtin_amdgcn_exp2f(fmaf(x[v], c, -rs))) * sc;
        cm[u] = lm;
    }
#pragma unroll
    for (int u = 0; u < N; ++u) cm[u] = wave_sum(cm[u]);  // independent reductions
    // (VEC: a chunk is one tile, so these equal the tile totals the element
    // scan forms; scalar: the chunk's four tiles summed in one go)
    int32_t ch = -1, last = -1;
    double cb = 0.0, last_b = 0.0, run = before;
#pragma unroll
    for (int u = 0; u < N; ++u) {
        if (ch < 0 && cm[u] > 0.0) {
            if (run <= target && target < run + cm[u]) {
                ch = u;
                cb = run;
            }
            last = u;
            last_b = run;
        }
        run += cm[u];
    }
    if (ch < 0) {
        ch = last;
        cb = last_b;
    }
    int32_t tok = -1;
#pragma unroll
    for (int u = 0; u < N; ++u)  // (a branch per chunk keeps the register indices constant)
        if (ch == u) tok = draft_pick<DT, VEC, 1>(q + u, c0 + u, c, rs, sc, cb, target, lane, mass);
    return tok;
}

template <int DT, bool VEC, bool GREEDY, bool ENT>
__device__ inline void draft_finish(const DraftParams& D, int64_t row, int lane);

template <int DT, bool VEC, bool GREEDY, bool ENT>
__global__ __launch_bounds__(kBlock) void k_draft(DraftParams D) {
    using C = Chunk<DT, VEC>;
    using Raw = typename C::Raw;
    const int lane = static_cast<int>(threadIdx.x & (kWave - 1));
    const int w = static_cast<int>(__builtin_amdgcn_readfirstlane(threadIdx.x / kWave));  // (uniform: scalar branches)
    const int64_t sblocks = D.rows * D.nbr;
    if (blockIdx.x >= sblocks) {  // closing blocks: wavefront w finishes one row
        const int64_t row = (blockIdx.x - sblocks) * kWavesPerBlock + w;
        if (row < D.rows) draft_finish<DT, VEC, GREEDY, ENT>(D, row, lane);
        return;
    }
    const int64_t row = blockIdx.x / D.nbr;
    const int32_t wl = static_cast<int32_t>(blockIdx.x - row * D.nbr) * kWavesPerBlock + w;
    const char* rp = row_at<DT>(D.logits, row * D.V);
    const int64_t pb = row * D.nw;  // the row's partials
    if (wl < D.nw) {
        const int64_t c0 = static_cast<int64_t>(wl) * kDraftCw;
        Raw q[kDraftCw];
        load_slots<DT, VEC, kDraftCw>(q, rp, c0, D.nchunk, D.V, lane);
        mask_slots<DT, VEC, kDraftCw>(q, c0, D.nchunk, D.V, lane);
        if constexpr (GREEDY) {
            ArgLane a;
            a.init();
#pragma unroll
            for (int g = 0; g < kDraftCw / kUnroll; ++g)  // ascending: the first maximum is kept
                consume_group<DT, VEC, kUnroll>(a, q + g * kUnroll, c0 + g * kUnroll, lane, 0.0f);
            const bool nan = __ballot(a.nan) != 0;
            ArgPart f{a.best, a.at};
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) f = fold_arg(f, ArgPart{__shfl_xor(f.m, o, kWave), __shfl_xor(f.at, o, kWave)});
            if (lane == 0) {
                uint64_t* pw = D.part + (pb + wl) * kDraftWords;
                cst64(pw, tagged(D.epoch, __float_as_uint(nan ? NAN : f.m)));
                cst64(pw + 1, tagged(D.epoch, static_cast<uint32_t>(f.at)));
            }
        } else {
            // one pass: the reference R comes from the first group with a
            // finite maximum; a later group whose fp32 sum overflows (a value
            // far above R, or +inf) or is NaN takes the rare path, which
            // raises R (rescaling the sum so far by an exact power of two) and
            // sums the group again
            const float c = D.c32;
            float R = kRUnset;
            bool bad = false;
            double S = 0.0, SH = 0.0;  // (SH: sum of 2^t * t, for the entropy)
            auto sums = [&](const Raw* qg, float& acc, float& acc_t) {
                if constexpr (ENT) group_exp_tsum<DT, VEC, kUnroll>(qg, c, R, acc, acc_t);
                else acc = group_exp_sum<DT, VEC, kUnroll>(qg, c, R);
            };
#pragma unroll
            for (int g = 0; g < kDraftCw / kUnroll; ++g) {
                const Raw* qg = q + g * kUnroll;
                if (R == kRUnset) {
                    const float mx = wave_max(group_max<DT, VEC, kUnroll>(qg));  // (NaN is not a maximum)
                    if (mx * c > kRUnset + 1.0f) {
                        const float Rn = ceilf(mx * c);
                        if (Rn < 3.0e38f) R = Rn;
                        else bad = true;  // +inf logit, or x*c overflows: the row is unusable
                    }
                }
                float acc = 0.0f, acc_t = 0.0f;
                sums(qg, acc, acc_t);
                if (__any(!(acc <= 3.0e38f))) {
                    const float Rn = ceilf(wave_max(group_max<DT, VEC, kUnroll>(qg)) * c);
                    if (!(Rn < 3.0e38f)) {
                        bad = true;
                    } else if (Rn > R) {
                        // t shifts by R - Rn and every mass scales by 2^(R - Rn)
                        if constexpr (ENT) SH = S == 0.0 ? 0.0 : rebase(SH + static_cast<double>(R - Rn) * S, R, Rn);
                        S = rebase(S, R, Rn);
                        R = Rn;
                        sums(qg, acc, acc_t);
                    }  // else a NaN logit: the sum stays NaN
                }
                S += static_cast<double>(acc);
                if constexpr (ENT) SH += static_cast<double>(acc_t);
            }
            S = wave_sum(S);
            if constexpr (ENT) SH = wave_sum(SH);
            if (lane == 0) {
                uint64_t* pw = D.part + (pb + wl) * kDraftWords;
                cst64(pw, tagged(D.epoch, __float_as_uint(bad ? NAN : static_cast<float>(S))));
                cst64(pw + 1, tagged(D.epoch, __float_as_uint(R)));
                if constexpr (ENT) cst64(pw + 2, tagged(D.epoch, __float_as_uint(static_cast<float>(SH))));
            }
        }
    }
    // (the tagged words are this range's arrival: nothing else to count)
}

// The closing wavefront of a row: waits (bounded) until all of the row's
// ranges have counted in, clears the counter for the next call, and draws.
// The closing wavefront of a row: reads the row's tagged range words until
// every one carries this call's epoch (bounded), then draws. Rows of at most
// kFinTiles * 64 ranges keep the words of the read that found them all
// current, so a row that is already complete costs one round trip here.
template <int DT, bool VEC, bool GREEDY, bool ENT>
__device__ inline void draft_finish(const DraftParams& D, int64_t row, int lane) {
    using C = Chunk<DT, VEC>;
    using Raw = typename C::Raw;
    const int32_t nw = D.nw;
    const uint64_t* pw = D.part + row * nw * kDraftWords;
    constexpr int NWD = GREEDY ? 2 : (ENT ? 3 : 2);  // words per range in use
    const uint32_t ep = D.epoch;
    auto current = [&](uint64_t e) { return static_cast<uint32_t>(e >> 32) == ep; };
    auto f32 = [](uint64_t e) { return __uint_as_float(static_cast<uint32_t>(e)); };
    const bool hold = nw <= kFinTiles * kWave;
    uint64_t e[kFinTiles][3];
    bool ok = true;
    {
        const uint64_t t0 = wall_clock64();
        for (;;) {
            bool stale = false;
            if (hold) {
#pragma unroll
                for (int t = 0; t < kFinTiles; ++t) {
                    const int32_t k = t * kWave + lane;
#pragma unroll
                    for (int wd = 0; wd < 3; ++wd) {
                        e[t][wd] = k < nw && wd < NWD ? cld64(pw + static_cast<int64_t>(k) * kDraftWords + wd)
                                                      : tagged(ep, 0u);
                        stale |= !current(e[t][wd]);
                    }
                }
            } else {
                for (int32_t k = lane; k < nw; k += kWave)
                    for (int wd = 0; wd < NWD; ++wd) stale |= !current(cld64(pw + static_cast<int64_t>(k) * kDraftWords + wd));
            }
            if (__ballot(stale) == 0) break;
            if (wall_clock64() - t0 > D.wait) {
                // (the range words are tagged with the call's epoch, so nothing
                // needs draining: the row is reported unusable)
                if (lane == 0) cst(D.err, 1u);
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(kSleep);
        }
    }
    after_complete();
    if (!ok) {  // the wait ran out: the row is reported unusable
        if (lane == 0) {
            D.out_tokens[row] = -1;
            if (D.out_q) D.out_q[row] = NAN;
            if (D.out_h) D.out_h[row] = NAN;
        }
        return;
    }
    // (a range's words, from the held read or from memory; all current now)
    auto word = [&](int32_t k, int wd) { return cld64(pw + static_cast<int64_t>(k) * kDraftWords + wd); };
    const char* rp = row_at<DT>(D.logits, row * D.V);
    if constexpr (GREEDY) {
        ArgPart f{-INFINITY, INT32_MAX};
        if (hold) {
#pragma unroll
            for (int t = 0; t < kFinTiles; ++t)
                if (t * kWave + lane < nw) f = fold_arg(f, ArgPart{f32(e[t][0]), static_cast<int32_t>(e[t][1])});
        } else {
            for (int32_t k = lane; k < nw; k += kWave)
                f = fold_arg(f, ArgPart{f32(word(k, 0)), static_cast<int32_t>(word(k, 1))});
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) f = fold_arg(f, ArgPart{__shfl_xor(f.m, o, kWave), __shfl_xor(f.at, o, kWave)});
        if (lane == 0) {
            const bool good = isfinite(f.m);
            D.out_tokens[row] = good ? f.at : -1;
            if (D.out_q) D.out_q[row] = good ? 1.0 : static_cast<double>(NAN);
            if (D.out_h) D.out_h[row] = good ? 0.0 : static_cast<double>(NAN);  // a point mass
        }
    } else {
        // the ranges' sums at the row's reference R (an exact power-of-two
        // rescaling of each range's own), their total S, the range where the
        // ascending cumulative mass crosses u*S; then that range again, and
        // the element in it
        double S = 0.0, SH = 0.0, before = 0.0, target = 0.0;
        float R = kRUnset, rs = kRUnset;
        int32_t sel = -1;
        const int64_t b = row / D.n, t = row - b * D.n;
        const double u = philox_uniform(D.seed, static_cast<uint32_t>(b + D.b_offset),
                                        static_cast<uint32_t>(D.pos0 + t), kPurposeDraft);
        // a range's sum of 2^t * t at the row's reference: 2^(r - R) * (h + (r - R) * s)
        auto sh_at = [&](double h, double sv, float r) {
            return sv == 0.0 ? 0.0 : rebase(h, r, R) + static_cast<double>(r - R) * rebase(sv, r, R);
        };
        if (hold) {
            float r[kFinTiles];
            double v[kFinTiles], incl[kFinTiles];
#pragma unroll
            for (int t2 = 0; t2 < kFinTiles; ++t2) {
                const bool in = t2 * kWave + lane < nw;
                r[t2] = in ? f32(e[t2][1]) : kRUnset;
                v[t2] = in ? static_cast<double>(f32(e[t2][0])) : 0.0;
            }
#pragma unroll
            for (int t2 = 0; t2 < kFinTiles; ++t2) R = fmaxf(R, r[t2]);
            R = wave_max(R);
            if constexpr (ENT) {
                double sh = 0.0;
#pragma unroll
                for (int t2 = 0; t2 < kFinTiles; ++t2)
                    if (t2 * kWave + lane < nw) sh += sh_at(static_cast<double>(f32(e[t2][2])), v[t2], r[t2]);
                SH = wave_sum(sh);
            }
#pragma unroll
            for (int t2 = 0; t2 < kFinTiles; ++t2) v[t2] = rebase(v[t2], r[t2], R);
            const int nt = static_cast<int>((nw + kWave - 1) / kWave);
            S = regs_scan<kFinTiles>(v, incl, lane, nt);
            if (isfinite(S) && S > 0.0) {  // else NaN, +inf or no finite entry: the row is unusable
                target = u * S;
                sel = regs_find<kFinTiles>(v, incl, target, lane, before, nt);
                if (sel >= 0) {
#pragma unroll
                    for (int t2 = 0; t2 < kFinTiles; ++t2)
                        if (sel / kWave == t2) rs = r[t2];  // (constant register indices)
                    rs = __shfl(rs, sel % kWave, kWave);
                }
            }
        } else {  // many ranges: three passes over them in tiles of 64
            for (int32_t t0 = 0; t0 < nw; t0 += kWave)
                if (t0 + lane < nw) R = fmaxf(R, f32(word(t0 + lane, 1)));
            R = wave_max(R);
            auto val = [&](int32_t k) {
                return k < nw ? rebase(static_cast<double>(f32(word(k, 0))), f32(word(k, 1)), R) : 0.0;
            };
            for (int32_t t0 = 0; t0 < nw; t0 += kWave) S += lane_f64(wave_scan_incl(val(t0 + lane)), kWave - 1);
            if constexpr (ENT) {
                for (int32_t t0 = 0; t0 < nw; t0 += kWave) {
                    const int32_t k = t0 + lane;
                    SH += wave_sum(k < nw ? sh_at(static_cast<double>(f32(word(k, 2))),
                                                  static_cast<double>(f32(word(k, 0))), f32(word(k, 1)))
                                          : 0.0);
                }
            }
            if (isfinite(S) && S > 0.0) {
                target = u * S;
                double base = 0.0, last_before = 0.0;
                int32_t last = -1;
                for (int32_t t0 = 0; t0 < nw && sel < 0; t0 += kWave) {
                    const double v = val(t0 + lane);
                    const double incl = base + wave_scan_incl(v);
                    const double prev = lane_before(incl);
                    const double excl = lane == 0 ? base : prev;
                    const uint64_t hit = __ballot(v > 0.0 && excl <= target && target < incl);
                    if (hit) {
                        const int l = __ffsll(static_cast<unsigned long long>(hit)) - 1;
                        sel = t0 + l;
                        before = __shfl(excl, l, kWave);
                    } else {
                        const uint64_t any = __ballot(v > 0.0);
                        if (any) {
                            const int l = 63 - __clzll(static_cast<unsigned long long>(any));
                            last = t0 + l;
                            last_before = __shfl(excl, l, kWave);
                        }
                    }
                    base = lane_f64(incl, kWave - 1);
                }
                if (sel < 0) {
                    sel = last;
                    before = last_before;
                }
                if (sel >= 0) rs = f32(word(sel, 1));
            }
        }
        int32_t tok = -1;
        double qv = NAN;
        if (sel >= 0) {
            const int64_t c0 = static_cast<int64_t>(sel) * kDraftCw;
            Raw q[kDraftCw];
            load_slots<DT, VEC, kDraftCw>(q, rp, c0, D.nchunk, D.V, lane);
            mask_slots<DT, VEC, kDraftCw>(q, c0, D.nchunk, D.V, lane);
            const double sc = ldexp(1.0, static_cast<int>(fmaxf(rs - R, -1100.0f)));
            double mass = 0.0;
            tok = draft_pick_range<DT, VEC, kDraftCw>(q, c0, D.c32, rs, sc, before, target, lane, mass);
            if (tok >= 0) qv = mass / S;
        }
        if (lane == 0) {
            D.out_tokens[row] = tok;
            if (D.out_q) D.out_q[row] = qv;
            // H = -sum p ln p with p = 2^t / S: ln S - ln 2 * (sum 2^t t) / S
            if (ENT && D.out_h)
                D.out_h[row] = isfinite(S) && S > 0.0 ? log(S) - 0.69314718055994530942 * SH / S : static_cast<double>(NAN);
        }
    }
}

// ==========================================================================
// Expected acceptance per position (Lemma 1 of [Ch15] 15.1.2: a draft token
// drawn from q_i is accepted with probability beta_i = sum_x min(p_i(x),
// q_i(x))), the diagnostic behind the acceptance-rate rule for the draft
// length ([Ch15] 15.1.4, dynamic strategy adjustment). Given each row's
// (max m, S = sum exp((l - m)/T)) from the statistics pass, p_j = 2^(fl(x_j*c)
// - mc) * sp with mc = fl(m*c) and sp = 2^(mc - m*c)/S (likewise q). One
// launch: wavefront ranges of kDraftCw chunks of both rows of a pair sum
// min(p_j, q_j) (fp32 per load group, fp64 across); a closing wavefront per
// pair adds the ranges in order.
// ==========================================================================
// Overlap blocks trail their pair's statistics blocks by this many pairs in
// the grid: about two chip-fulls of blocks, so the statistics are done when
// the overlap blocks start, while the rows read in between (about 66 MB at
// the headline shape) stay well below the 256 MB memory-side cache. Chosen
// by timing on the headline shape (lag 64: 122 us; 128: 91; 192: 91; 256:
// 92; 384: 95; all statistics first: 98, against 103 with non-temporal loads).
#ifndef SPECVERIFY_OVERLAP_LAG
#define SPECVERIFY_OVERLAP_LAG 128
#endif
constexpr int64_t kOverlapLag = SPECVERIFY_OVERLAP_LAG;

struct OverlapParams {
    const void* tgt;  // [B, gamma + 1, V]
    const void* dft;  // [B, gamma, V]
    int32_t B, gamma, V, nchunk, nw, nbr;
    float c32;
    const float* m_t;   // row maxima and sums: pair p's target row at [2p], its draft row at [2p + 1]
    const double* s_t;
    double* part;       // [pairs, nw]
    uint32_t* cnt;      // [pairs] counters, kDraftStride words apart
    uint32_t* err;
    double* out_beta;   // [B * gamma]
    int64_t sbp;           // row-statistics blocks per pair (its target row's, then its draft row's)
    int64_t lag;           // pairs between a pair's statistics blocks and its overlap blocks
    uint32_t* rows_done;   // [pairs] finished rows of the pair (two), kSyncStride words apart
    uint64_t wait;         // bound on a wait, in wall-clock ticks
};

template <int DT, bool VEC>
__device__ inline void overlap_finish(const OverlapParams& O, int64_t pair, int lane) {
    uint32_t* cnt = O.cnt + pair * kDraftStride;
    const uint32_t want = static_cast<uint32_t>(O.nw);
    int ok = 1;
    if (lane == 0) {
        auto all_in = [&] { return cld(cnt) >= want; };
        bool drained = true;
        if (!spin_until(all_in, O.wait)) {  // the pair is reported NaN; drain before resetting
            cst(O.err, 1u);
            ok = 0;
            drained = spin_until(all_in, kWaitTicks);
        }
        if (drained) {  // every range of the pair has counted in, each after its rows were finished
            cst(cnt, 0u);
            cst(O.rows_done + pair * kSyncStride, 0u);
        }
    }
    ok = __shfl(ok, 0, kWave);
    after_complete();
    double acc = 0.0;
    for (int32_t k = lane; k < O.nw; k += kWave) acc += cld(O.part + pair * O.nw + k);
    acc = wave_sum(acc);
    if (lane == 0) O.out_beta[pair] = ok ? acc : static_cast<double>(NAN);
}

// One launch. Each pair has sbp row-statistics blocks (its target row's, then
// its draft row's; each row's finisher counts the row in at the pair) and nbr
// overlap blocks, whose wavefronts wait (bounded) until both rows of their
// pair are finished and then read the rows again. The overlap blocks of pair
// p come lag pairs after its statistics blocks in the grid (statistics of
// pairs [0, lag); then for each later pair t its statistics followed by the
// overlap blocks of pair t - lag; then the overlap blocks of the last lag
// pairs), so the second read follows the first by about lag pairs' rows and
// finds them in the memory-side cache; the closing blocks come last. A block
// waits only for blocks before it in the grid, which in-order dispatch has
// started, so no wait depends on a block that cannot start.
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_overlap(Params P, OverlapParams O) {
    using C = Chunk<DT, VEC>;
    using Raw = typename C::Raw;
    const int64_t pairs = static_cast<int64_t>(O.B) * O.gamma;
    const int64_t SB = O.sbp, R = O.nbr, D = O.lag;
    int64_t x = static_cast<int64_t>(blockIdx.x);
    int64_t pair, idx;
    bool stats = false;
    const int64_t head = D * SB, mid = (pairs - D) * (SB + R), tail = D * R;
    if (x < head) {
        stats = true;
        pair = x / SB;
        idx = x - pair * SB;
    } else if ((x -= head) < mid) {
        const int64_t t = x / (SB + R), o = x - t * (SB + R);
        stats = o < SB;
        pair = stats ? D + t : t;
        idx = stats ? o : o - SB;
    } else if ((x -= mid) < tail) {
        pair = pairs - D + x / R;
        idx = x - (x / R) * R;
    } else {
        x -= tail;
        pair = -1;
        idx = x;
    }
    if (stats) {
        stats_block<DT, VEC, kRows, false>(P, role_at<kRows>(P, static_cast<uint32_t>(pair * SB + idx)));
        return;
    }
    const int lane = static_cast<int>(threadIdx.x & (kWave - 1));
    const int w = static_cast<int>(__builtin_amdgcn_readfirstlane(threadIdx.x / kWave));
    if (pair < 0) {  // closing blocks: wavefront w finishes one pair
        const int64_t p = idx * kWavesPerBlock + w;
        if (p < pairs) overlap_finish<DT, VEC>(O, p, lane);
        return;
    }
    const int32_t wl = static_cast<int32_t>(idx) * kWavesPerBlock + w;
    if (wl >= O.nw) return;
    const int64_t b = pair / O.gamma, i = pair - b * O.gamma;
    const int64_t rt = b * (O.gamma + 1) + i;
    // the pair's two rows are finished once its count reaches two
    int ready = 1;
    if (lane == 0) {
        const uint32_t* rd = O.rows_done + pair * kSyncStride;
        auto both = [&] { return cld(rd) >= 2u; };
        if (!spin_until(both, O.wait)) {
            // the pair is reported NaN; the rows are still awaited (drained), so
            // that the pair's finisher resets their count only after both came
            cst(O.err, 1u);
            ready = 0;
            (void)spin_until(both, kWaitTicks);
        }
    }
    ready = __shfl(ready, 0, kWave);
    after_complete();
    const float c = O.c32;
    const float mp = cld(O.m_t + 2 * pair), mq = cld(O.m_t + 2 * pair + 1);
    const double Sp = cld(O.s_t + 2 * pair), Sq = cld(O.s_t + 2 * pair + 1);
    const bool ok = ready && isfinite(Sp) && isfinite(Sq) && Sp > 0.0 && Sq > 0.0;
    const float mcp = mp * c, mcq = mq * c;
    const float sp = ok ? static_cast<float>(exp2(static_cast<double>(mcp) - static_cast<double>(mp) * c) / Sp) : 0.0f;
    const float sq = ok ? static_cast<float>(exp2(static_cast<double>(mcq) - static_cast<double>(mq) * c) / Sq) : 0.0f;
    const int64_t c0 = static_cast<int64_t>(wl) * kDraftCw;
    Raw qp[kDraftCw], qq[kDraftCw];
    load_slots<DT, VEC, kDraftCw, false>(qp, row_at<DT>(O.tgt, rt * O.V), c0, O.nchunk, O.V, lane);
    load_slots<DT, VEC, kDraftCw, false>(qq, row_at<DT>(O.dft, pair * O.V), c0, O.nchunk, O.V, lane);
    mask_slots<DT, VEC, kDraftCw>(qp, c0, O.nchunk, O.V, lane);
    mask_slots<DT, VEC, kDraftCw>(qq, c0, O.nchunk, O.V, lane);
    double S = 0.0;
#pragma unroll
    for (int u = 0; u < kDraftCw; ++u) {
        float xp[C::EPL], xq[C::EPL];
        C::expand(qp[u], xp);
        C::expand(qq[u], xq);
        float a = 0.0f;
#pragma unroll
        for (int v = 0; v < C::EPL; ++v)
            a += fminf(__builtin_amdgcn_exp2f(fmaf(xp[v], c, -mcp)) * sp, __builtin_amdgcn_exp2f(fmaf(xq[v], c, -mcq)) * sq);
        S += static_cast<double>(a);
    }
    S = wave_sum(S);
    if (lane == 0) cst(O.part + pair * O.nw + wl, ok ? S : static_cast<double>(NAN));
    complete_before();
    if (lane == 0)
        (void)__hip_atomic_fetch_add(O.cnt + pair * kDraftStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ==========================================================================
// Token-tree verification, a labelled heuristic mode ([CSDN] 3.2
// TokenTreeVerifier.parallel_verify; [Ch15] 15.2.4 candidate trees). Not
// distribution-preserving: from the root, the children of the last accepted
// node are scored by the acceptance probability min(1, p/q) of their tokens
// under the parent's target and draft rows (T == 0: 1 for the child whose
// token is the parent row's target argmax), the first child with the largest
// score is taken while it reaches the threshold. The rows' statistics (or
// argmaxes) come from the statistics kernels over every node's rows; the walk
// itself is one wavefront per sequence gathering two logits per child.
// ==========================================================================
struct TreeParams {
    const void* tgt;       // [B, N, V]
    const void* dft;       // [B, N, V] (T > 0)
    const int32_t* parent; // [B, N]
    const int32_t* token;  // [B, N]
    int32_t B, N, V;
    double T;              // the temperature (0: greedy)
    double threshold;
    const float* m_t;      // [B * N] row maxima and sums (T > 0)
    const double* s_t;
    const float* m_d;
    const double* s_d;
    const int32_t* amax;   // [B * N] target argmax per row, -1 if unusable (T == 0)
    int32_t* out_tokens;   // [B, N - 1]
    int32_t* out_nodes;    // [B, N - 1] or null
    int32_t* out_n;        // [B]
    // the fused launch: blocks from first_block on walk the trees; tree b's
    // rows are finished once done[b * kSyncStride] reaches 2N (reset by the walk)
    int64_t first_block;
    uint32_t* done;
    uint32_t* err;         // sticky: a wait ran out
    uint64_t wait;         // bound on the walk's wait, in wall-clock ticks
};

// Trees of at most kTreeHold * 64 nodes are loaded whole at the start (lane
// l, slot t: node 64 t + l): its parent and token, the statistics of its own
// rows, and the two logits of its token under its parent's rows. The walk is
// then register and cross-lane work only. Larger trees read the parent and
// token arrays and gather the logits at every level.
constexpr int kTreeHold = 4;

// The walk of tree b by one wavefront. FUSED (HOLD, T > 0): the statistics
// are produced by the same launch, so the parents, tokens and gathered logits
// are loaded first, then the wavefront waits (bounded) until the tree's 2N rows
// are finished and reads their statistics with coherent loads.
template <int DT, bool HOLD, bool FUSED>
__device__ inline void walk_tree(const TreeParams& Q, int64_t b, int lane) {
    static_assert(!FUSED || HOLD, "the fused walk holds the tree");
    const int32_t N = Q.N;
    const bool sample = Q.T > 0.0;
    const int32_t* par = Q.parent + b * N;
    const int32_t* tok = Q.token + b * N;
    int32_t* ot = Q.out_tokens + b * (N - 1);
    int32_t* on = Q.out_nodes ? Q.out_nodes + b * (N - 1) : nullptr;
    constexpr int NT = HOLD ? kTreeHold : 1;
    int32_t hp[NT], ht[NT], ham[NT];
    float hmt[NT], hmd[NT], glt[NT], gld[NT];
    double hst[NT], hsd[NT];
    if constexpr (HOLD) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int32_t j = t * kWave + lane;
            const bool in = j < N;
            const int64_t rj = b * N + j;
            hp[t] = in ? par[j] : -1;
            ht[t] = in ? tok[j] : -1;
            if constexpr (!FUSED) {
                hmt[t] = in && sample ? Q.m_t[rj] : 0.0f;
                hmd[t] = in && sample ? Q.m_d[rj] : 0.0f;
                hst[t] = in && sample ? Q.s_t[rj] : 0.0;
                hsd[t] = in && sample ? Q.s_d[rj] : 0.0;
                ham[t] = in && !sample ? Q.amax[rj] : -1;
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {  // the node's token under its parent's rows
            const int32_t j = t * kWave + lane;
            const bool ok = sample && j >= 1 && j < N && hp[t] >= 0 && hp[t] < j && ht[t] >= 0 && ht[t] < Q.V;
            const int64_t rp = (b * N + (ok ? hp[t] : 0)) * Q.V;
            glt[t] = ok ? load_one<DT>(row_at<DT>(Q.tgt, rp), ht[t]) : 0.0f;
            gld[t] = ok ? load_one<DT>(row_at<DT>(Q.dft, rp), ht[t]) : 0.0f;
        }
    }
    bool lost = false;  // FUSED: the wait for the tree's rows ran out
    if constexpr (FUSED) {
        uint32_t* cnt = Q.done + b * kSyncStride;
        const uint32_t want = 2u * static_cast<uint32_t>(N);
        auto all_in = [&] { return cld(cnt) == want; };
        bool drained = true;
        if (!spin_until(all_in, Q.wait)) {  // the tree is reported invalid; drain before resetting
            if (lane == 0) cst(Q.err, 1u);
            lost = true;
            drained = spin_until(all_in, kWaitTicks);
        }
        after_complete();
        if (drained && lane == 0) cst(cnt, 0u);  // every row of the tree has counted in
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int32_t j = t * kWave + lane;
            const bool in = j < N;
            const int64_t rj = b * N + j;
            hmt[t] = in ? cld(Q.m_t + rj) : 0.0f;
            hmd[t] = in ? cld(Q.m_d + rj) : 0.0f;
            hst[t] = in ? cld(Q.s_t + rj) : 0.0;
            hsd[t] = in ? cld(Q.s_d + rj) : 0.0;
            ham[t] = -1;
        }
    }
    // every node's score under its parent's rows (T > 0), computed once: the
    // parent's statistics come from the lane holding the parent, and the walk
    // then only compares (tiles past the last node are skipped)
    double hsc[NT];
    if constexpr (HOLD) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            hsc[t] = -2.0;
            if (!sample || t * kWave >= N) continue;
            const int32_t j = t * kWave + lane, pj = hp[t];
            const int src = pj >= 0 ? pj % kWave : 0;
            double pmt = 0.0, pmd = 0.0, pst = 0.0, psd = 0.0;
#pragma unroll
            for (int ts = 0; ts < NT; ++ts) {
                if (ts * kWave >= N) break;
                const float a = __shfl(hmt[ts], src, kWave), d = __shfl(hmd[ts], src, kWave);
                const double sa = __shfl(hst[ts], src, kWave), sd = __shfl(hsd[ts], src, kWave);
                if (pj >= 0 && pj / kWave == ts) {
                    pmt = a;
                    pmd = d;
                    pst = sa;
                    psd = sd;
                }
            }
            const bool node = j >= 1 && j < N && pj >= 0 && pj < j && ht[t] >= 0 && ht[t] < Q.V;
            if (node && isfinite(pst) && isfinite(psd) && pst > 0.0 && psd > 0.0) {
                const double pp = exp((static_cast<double>(glt[t]) - pmt) / Q.T) / pst;
                const double qq = exp((static_cast<double>(gld[t]) - pmd) / Q.T) / psd;
                hsc[t] = pp == 0.0 ? 0.0 : (qq == 0.0 ? 1.0 : fmin(1.0, pp / qq));
            }
        }
    }
    // every parent must come before its child
    bool bad = false;
    if constexpr (HOLD) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int32_t j = t * kWave + lane;
            bad |= j >= 1 && j < N && (hp[t] < 0 || hp[t] >= j);
        }
    } else {
        for (int32_t j = 1 + lane; j < N; j += kWave) bad |= par[j] < 0 || par[j] >= j;
    }
    bool invalid = __ballot(bad) != 0 || lost;
    int32_t v = 0, n = 0;
    while (!invalid) {
        const int64_t rv = b * N + v;
        double lmt = 0.0, lmd = 0.0, St = 0.0, Sd = 0.0;
        int32_t av = -1;
        if constexpr (HOLD) {  // node v's statistics from the lane holding v
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (v / kWave == t) {  // (constant register indices)
                    const int src = v % kWave;
                    lmt = __shfl(hmt[t], src, kWave);
                    lmd = __shfl(hmd[t], src, kWave);
                    St = __shfl(hst[t], src, kWave);
                    Sd = __shfl(hsd[t], src, kWave);
                    av = __shfl(ham[t], src, kWave);
                }
            }
        } else if (sample) {
            lmt = Q.m_t[rv];
            lmd = Q.m_d[rv];
            St = Q.s_t[rv];
            Sd = Q.s_d[rv];
        } else {
            av = Q.amax[rv];
        }
        const bool usable_v = sample ? isfinite(St) && isfinite(Sd) && St > 0.0 && Sd > 0.0 : av >= 0;
        // the children of v, 64 at a time: (score desc, index asc)
        double best_s = -2.0;
        int32_t best = INT32_MAX;
        bool any_child = false, bad_tok = false;
        auto visit = [&](int32_t j, bool child, int32_t x, float lt, float ld, double pre) {
            double sc = -2.0;
            if (child) {
                if (x < 0 || x >= Q.V) {
                    bad_tok = true;
                } else if (usable_v) {
                    if (sample) {
                        if constexpr (HOLD) {
                            sc = pre;
                        } else {
                            // acceptance probability in fp64 from the two logits of the child's token
                            const double p = exp((static_cast<double>(lt) - lmt) / Q.T) / St;
                            const double q = exp((static_cast<double>(ld) - lmd) / Q.T) / Sd;
                            sc = p == 0.0 ? 0.0 : (q == 0.0 ? 1.0 : fmin(1.0, p / q));
                        }
                    } else {
                        sc = x == av ? 1.0 : -1.0;
                    }
                }
            }
            any_child |= __ballot(child) != 0;
            // fold this tile's candidates into (best_s, best): a later tile
            // replaces the best only with a strictly larger score
            double tile_max = sc;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) tile_max = fmax(tile_max, __shfl_xor(tile_max, o, kWave));
            if (tile_max > best_s) {
                const uint64_t at = __ballot(child && sc == tile_max);
                best_s = tile_max;
                best = (j - lane) + (__ffsll(static_cast<unsigned long long>(at)) - 1);
            }
        };
        if constexpr (HOLD) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (t * kWave >= N) break;
                const int32_t j = t * kWave + lane;
                visit(j, j > v && j < N && hp[t] == v, ht[t], glt[t], gld[t], hsc[t]);
            }
        } else {
            for (int32_t t0 = v + 1; t0 < N; t0 += kWave) {
                const int32_t j = t0 + lane;
                const bool child = j < N && par[j] == v;
                const int32_t x = child ? tok[j] : 0;
                float lt = 0.0f, ld = 0.0f;
                if (child && sample && x >= 0 && x < Q.V && usable_v) {
                    lt = load_one<DT>(row_at<DT>(Q.tgt, rv * Q.V), x);
                    ld = load_one<DT>(row_at<DT>(Q.dft, rv * Q.V), x);
                }
                visit(j, child, x, lt, ld, 0.0);
            }
        }
        if (__ballot(bad_tok) != 0 || (any_child && !usable_v)) {
            invalid = true;
            break;
        }
        if (!any_child) break;
        if (sample ? best_s < Q.threshold : best_s < 1.0) break;
        int32_t tb = 0;
        if constexpr (HOLD) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                if (best / kWave == t) tb = __shfl(ht[t], best % kWave, kWave);  // (constant register indices)
        } else {
            tb = tok[best];
        }
        if (lane == 0) {
            ot[n] = tb;
            if (on) on[n] = best;
        }
        ++n;
        v = best;
    }
    for (int32_t j = lane; j < N - 1; j += kWave) {
        if (invalid || j >= n) {
            ot[j] = -1;
            if (on) on[j] = -1;
        }
    }
    if (lane == 0) Q.out_n[b] = invalid ? -1 : n;
}

template <int DT, bool HOLD>
__global__ __launch_bounds__(kBlock) void k_tree_walk(TreeParams Q) {
    const int lane = static_cast<int>(threadIdx.x & (kWave - 1));
    const int w = static_cast<int>(__builtin_amdgcn_readfirstlane(threadIdx.x / kWave));
    const int64_t b = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + w;
    if (b >= Q.B) return;
    walk_tree<DT, HOLD, false>(Q, b, lane);
}

// T > 0, trees of up to kTreeHold*64 nodes: one launch. Blocks before
// Q.first_block are the row-statistics blocks over every node's target rows,
// then its draft rows (each row's finisher counts the row in at its tree);
// the blocks after them hold one walking wavefront per tree. They come last in
// the grid, so every statistics block has started before any of them waits.
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_tree(Params P, TreeParams Q) {
    if (static_cast<int64_t>(blockIdx.x) < Q.first_block) {
        stats_block<DT, VEC, kRows>(P, role_of<kRows>(P));
        return;
    }
    const int lane = static_cast<int>(threadIdx.x & (kWave - 1));
    const int w = static_cast<int>(__builtin_amdgcn_readfirstlane(threadIdx.x / kWave));
    const int64_t b = (static_cast<int64_t>(blockIdx.x) - Q.first_block) * kWavesPerBlock + w;
    if (b >= Q.B) return;
    walk_tree<DT, true, true>(Q, b, lane);
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
// partial slots and residual block masses, laid out per call shape. `sync`
// holds the counters, the decision words, the draw records and the error word
// at fixed addresses: it is cleared when allocated, every call leaves its
// counters at zero again, and decision words and draw records are told apart
// by the call's epoch, so calls of any shape can follow one another on it.
struct Workspace {
    void* data = nullptr;
    size_t bytes = 0;
    uint32_t* sync = nullptr;
    int64_t cnt_cap = 0;  // counter words
    int64_t dec_cap = 0;  // decision words and draw records (64-bit)
    int64_t tag_cap = 0;  // epoch-tagged range words of the draft sampler (64-bit)
    uint32_t epoch = 0;   // of the last call
};

std::mutex g_mu;
std::map<std::pair<int, void*>, Workspace> g_ws;  // (device, stream) -> buffers
std::map<int, int> g_cus;                         // device -> compute units
std::atomic<int64_t> g_wait_limit{-1};            // host-set bound on a wait (ticks); < 0: kWaitTicks

uint64_t wait_ticks() {
    const int64_t v = g_wait_limit.load(std::memory_order_relaxed);
    return v < 0 ? kWaitTicks : static_cast<uint64_t>(v);
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Layout {
    Params p;  // geometry filled; pointers added at launch
    bool group;      // the group-major kernel (else the position-major one)
    int64_t units;
    int64_t blocks;
    uint32_t lds;    // dynamic LDS of the group-major kernel
    size_t off_pm, off_pr, off_ps, off_pi, off_tok, off_msum, off_subr, off_subR, bytes;
    int64_t cnt_words, dec_words;
    int64_t tag_words;  // epoch-tagged 64-bit words of the draft sampler's ranges
};

int elem_bytes(int32_t dtype) { return dtype == SPEC_F32 ? 4 : 2; }

// Chunk geometry: vector chunks are 1 KiB; scalar chunks are 64 x 4 elements.
int32_t chunk_elems(int32_t dtype, bool vec) { return vec ? kWave * (16 / elem_bytes(dtype)) : kWave * 4; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Statistics wavefronts take about kChunksPerWave chunks (16 at T == 0; many more wavefronts
// than the chip holds at once), but the whole problem gets at least 16
// wavefronts per compute unit so that small problems still spread over the
// chip. Residual wavefronts hold kPairCw chunks of each of the two rows.
Layout plan(int mode, int64_t G, int32_t gamma, int32_t V, int32_t dtype, bool vec, int cus) {
    Layout L{};
    Params& p = L.p;
    p.B = static_cast<int32_t>(G);
    p.gamma = gamma;
    p.V = V;
    const int32_t CH = chunk_elems(dtype, vec);
    p.nchunk = static_cast<int32_t>(ceil_div(V, CH));
    const int64_t rows = mode == kSample ? G * (2 * gamma + 1) : (mode == kGreedy ? G * (gamma + 1) : G);
    const int64_t total = rows * p.nchunk;
    const int64_t min_waves = static_cast<int64_t>(cus) * 16;
    int64_t cpw = mode != kGreedy ? kChunksPerWave : dtype == SPEC_BF16 ? kGreedyChunksPerWaveBf16 : kGreedyChunksPerWave;
    if (ceil_div(total, cpw) < min_waves) cpw = ceil_div(total, min_waves);
    // but long enough that a row has at most one wavefront's worth of slots
    // (the unit's fold takes a round trip per 64 slots of a row). Measured on
    // the greedy recipe: 7.15 against 8.35 us at B = 1, 7.5 against 8.4 at
    // 2, 8.9 against 9.45 at 4, unchanged from 8 on.
    cpw = std::max<int64_t>(cpw, ceil_div(p.nchunk, kWave - 1));
    if (cpw < 1) cpw = 1;
    p.cpw = static_cast<int32_t>(cpw);
    p.maxp = static_cast<int32_t>(ceil_div(p.nchunk, cpw) + 1);
    p.nw2 = mode == kSample ? static_cast<int32_t>(ceil_div(2 * static_cast<int64_t>(p.nchunk), cpw)) : 0;
    p.nb2 = static_cast<int32_t>(ceil_div(p.nw2, kWavesPerBlock));
    p.nw1 = static_cast<int32_t>(ceil_div(p.nchunk, cpw));
    p.nb1 = static_cast<int32_t>(ceil_div(p.nw1, kWavesPerBlock));
    p.nbr = mode == kSample ? static_cast<int32_t>(ceil_div(ceil_div(p.nchunk, kPairCw), kWavesPerBlock)) : 0;
    p.cstride = mode == kRows ? 1 : kSyncStride;
    L.units = mode == kRows ? G : G * (gamma + 1);
    p.rows_split = G;  // (row statistics: every row from tgt unless the caller splits)
    L.blocks = mode == kSample ? G * (static_cast<int64_t>(gamma) * p.nb2 + p.nb1 + p.nbr) : L.units * p.nb1;
    const size_t slots = static_cast<size_t>(L.units) * 2 * p.maxp;
    size_t o = 0;
    L.off_pm = o;
    o = align_up(o + slots * sizeof(float), 256);
    L.off_pr = o;
    o = align_up(o + (mode == kGreedy ? 0 : slots) * sizeof(float), 256);
    L.off_ps = o;
    o = align_up(o + (mode == kGreedy ? 0 : slots) * sizeof(double), 256);
    L.off_pi = o;
    o = align_up(o + (mode == kGreedy ? slots : 0) * sizeof(int32_t), 256);
    L.off_tok = o;
    o = align_up(o + (mode == kSample ? static_cast<size_t>(L.units) * 2 : 0) * sizeof(float), 256);
    L.off_msum = o;
    o = align_up(o + static_cast<size_t>(G) * p.nbr * kWavesPerBlock * sizeof(double), 256);
    L.bytes = o;
    L.cnt_words = L.units * p.cstride;
    L.dec_words = mode == kRows ? 0 : G * (gamma + 1) + (mode == kSample ? G * kRecWords : 0);
    return L;
}

// Group-major layout (T > 0): a group is one sequence's 2*gamma+1 rows (with
// `defer`, the statistics stream 2*gamma of them and the bonus row is left to
// the closing blocks), its statistics wavefronts take about
// kGroupChunksPerWave chunks each (at least 16 wavefronts per compute unit over
// the whole problem), and its residual wavefronts take spw subsegments of row
// k each.
Layout plan_group(int64_t G, int32_t gamma, int32_t V, int32_t dtype, bool vec, int cus, int mode = kSample,
                  bool defer = false, int32_t p0 = 0) {
    Layout L{};
    Params& p = L.p;
    L.group = true;
    const bool greedy = mode == kGreedy;  // the target rows only, and one closing block per group
    p.B = static_cast<int32_t>(G);
    p.gamma = gamma;
    p.V = V;
    p.rps = greedy ? gamma + 1 : 2 * gamma + 1;
    p.defer = defer && !greedy ? 1 : 0;
    p.srows = p.rps - p.defer;
    const int32_t CH = chunk_elems(dtype, vec);
    p.nchunk = static_cast<int32_t>(ceil_div(V, CH));
    const int64_t per_group = static_cast<int64_t>(p.srows) * p.nchunk;
    const int64_t min_waves = static_cast<int64_t>(cus) * 16;
    int64_t cpw = kGroupChunksPerWave;
    if (ceil_div(G * per_group, cpw) < min_waves) cpw = ceil_div(G * per_group, min_waves);
    // but not so short that a group's partial slots (rps rows of
    // ceil(nchunk / cpw) + 1) overflow the LDS stage: a fold from memory takes
    // one round trip per 8 slots of a row. Measured on the headline recipe:
    // 18.6 against 56.6 us at B = 1, 20.0 against 36.3 at 2, 21.7 against
    // 26.6 at 4 (from B = 8 on the ranges are long enough already).
    {
        const int64_t per_row = kMaxStage / p.rps - 1;
        if (per_row >= 1) cpw = std::max<int64_t>(cpw, ceil_div(p.nchunk, per_row));
    }
    if (cpw > static_cast<int64_t>(kMaxPieces - 1) * p.nchunk) cpw = static_cast<int64_t>(kMaxPieces - 1) * p.nchunk;
    if (cpw < 1) cpw = 1;
    p.cpw = static_cast<int32_t>(cpw);
    // two phases (T > 0, bonus row deferred, 0 < p0 < gamma): the first
    // phase's pairs, then the rest, each cut into ranges of its own
    p.p0 = !greedy && p.defer && p0 > 0 && p0 < gamma ? p0 : 0;
    const int64_t per_group1 = p.p0 ? 2 * static_cast<int64_t>(p.p0) * p.nchunk : per_group;
    p.nw = static_cast<int32_t>(ceil_div(per_group1, cpw));
    p.sb = static_cast<int32_t>(ceil_div(p.nw, kWavesPerBlock));
    // the second phase's ranges: longer from kLongPhase2Groups groups on
    // (fewer blocks wait for their group's decision while holding slots)
    {
        int64_t c2 = G >= kLongPhase2Groups ? std::max<int64_t>(cpw, kPhase2ChunksPerWave) : cpw;
        if (c2 > static_cast<int64_t>(kMaxPieces - 1) * p.nchunk) c2 = static_cast<int64_t>(kMaxPieces - 1) * p.nchunk;
        p.cpw2 = static_cast<int32_t>(c2);
    }
    p.pnw2 = p.p0 ? static_cast<int32_t>(ceil_div(2 * static_cast<int64_t>(gamma - p.p0) * p.nchunk, p.cpw2)) : 0;
    p.psb2 = static_cast<int32_t>(ceil_div(p.pnw2, kWavesPerBlock));
    p.maxp = static_cast<int32_t>(ceil_div(p.nchunk, cpw) + 1);
    p.nsub = static_cast<int32_t>(ceil_div(V, kSub));
    // residual subsegments per wavefront: one when the closing blocks of all
    // groups, so spread, come to between two and four per compute unit (the
    // chip then holds them all, each shorter), else as many as the kernel
    // holds in flight. Measured on the headline shape, one against two: 33.5
    // against 36.0 us at 32 groups (1024 closing blocks); 59.0 against 55.0 at
    // 64 groups (2048), 27.6 against 27.6 at 16 (512), 26.4 against 26.2 at 4,
    // and 17.4 against 16.9 on the 8-sequence fp32 workload (64).
    const int spw_max = vec ? (dtype == SPEC_BF16 ? subs_per_wave<SPEC_BF16, true>() : subs_per_wave<SPEC_F32, true>())
                            : subs_per_wave<SPEC_F32, false>();
    const int64_t closing1 = G * ceil_div(p.nsub, kWavesPerBlock);  // closing blocks at one subsegment each
    const int spw = closing1 > 2 * static_cast<int64_t>(cus) && closing1 <= 4 * static_cast<int64_t>(cus) ? 1 : spw_max;
    p.spw = spw;
    p.rb = greedy ? 1 : static_cast<int32_t>(ceil_div(p.nsub, kWavesPerBlock * spw));
    p.lag = static_cast<int32_t>(G < kLag ? G : kLag);
    if (p.p0) p.lag = static_cast<int32_t>(G > 2 * kDecideLag ? kDecideLag : G);
    {
        const int64_t group_bytes = static_cast<int64_t>(p.srows) * V * elem_bytes(dtype);
        const int64_t tail = greedy ? 0 : std::min<int64_t>(G, kCachedTailBytes / std::max<int64_t>(group_bytes, 1));
        p.cached_from = static_cast<int32_t>(G - tail);
    }
    p.cstride = kSyncStride;
    const int64_t gslots = static_cast<int64_t>(p.rps) * p.maxp;
    p.stage = gslots <= kMaxStage ? static_cast<int32_t>(gslots) : 0;
    L.units = G;
    L.blocks = G * (p.sb + p.rb) + (p.p0 ? G * (1 + p.psb2) : 0);
    L.lds = static_cast<uint32_t>(p.stage) * 20u;
    const size_t slots = static_cast<size_t>(G) * gslots;
    size_t o = 0;
    L.off_pm = o;
    o = align_up(o + slots * sizeof(float), 256);
    L.off_pr = o;
    o = align_up(o + (greedy ? 0 : slots) * sizeof(float), 256);
    L.off_ps = o;
    o = align_up(o + (greedy ? 0 : slots) * sizeof(double), 256);
    L.off_pi = o;
    o = align_up(o + (greedy ? slots : 0) * sizeof(int32_t), 256);
    L.off_tok = L.off_msum = o;
    L.off_subr = o;
    o = align_up(o + static_cast<size_t>(G) * p.nsub * sizeof(double), 256);
    L.off_subR = o;
    o = align_up(o + (p.defer ? static_cast<size_t>(G) * p.nsub * sizeof(float) : 0), 256);
    L.bytes = o;
    L.cnt_words = 2 * G * kSyncStride;
    // per group the word that marks its outputs void (a closing block's wait
    // ran out), then (two phases) the groups' decision records
    L.dec_words = G + (p.p0 ? G * kGroupRecWords : 0);
    return L;
}

// The automatic schedule at T > 0: position-major with the early stop once
// one position's row pairs come to at least kEarlyStopBytes (2 B V s):
// below that, decisions lag too many positions behind the stream to save
// reads; else group-major (in two phases where its rows are long enough,
// below). Measured, two phases against the early stop: on the headline
// recipe (V = 128256, bf16; 256.5 KB rows) 70.7 against 90.7 us at B = 128,
// 102.0 against 115.2 at 192, 131.5 against 139.7 at 256 (131 MB per
// position), 168.3 against 164.6 at 320 (164 MB), 200.2 against 190.4 at
// 384; on the 256-sequence recipe (V = 152064; 304 KB rows) 137.4 against
// 143.9 at B = 256 (156 MB), 173.1 against 168.7 at 320 (195 MB).
constexpr int64_t kEarlyStopBytes = int64_t(152) << 20;
bool auto_position_major(int64_t B, int32_t V, int32_t dtype) {
    // (B V stays below 2^62 for int32 shapes; the byte count may not)
    return B * static_cast<int64_t>(V) >= ceil_div(kEarlyStopBytes, 2 * static_cast<int64_t>(elem_bytes(dtype)));
}

// Two phases: the first phase's row pairs, about 3/8 of gamma (at least one,
// at most gamma - 1; 0 at gamma = 1: one phase). Measured with 1, 2, 3, 4
// pairs at gamma = 8 (headline recipe): 52.3, 47.7, 46.3, 47.3 us at B = 64,
// 71.0, 62.6, 58.1, 60.4 at B = 96; at gamma = 5 (8-sequence fp32 recipe,
// B = 256) 59.1, 54.6, 54.7, 67.0.
int32_t phase1_pairs(int32_t gamma) {
    if (gamma < 2) return 0;
    return std::max<int32_t>(1, std::min<int32_t>((3 * gamma + 4) / 8, gamma - 1));
}
// ... and only where the group-major stream is long enough for the rows it
// skips to outweigh the decider's step in the closing chain: at least this
// many bytes of the groups' rows (2 gamma B V s). Measured, two phases
// against one: on the headline recipe 30.4 against 30.1 us at B = 24 (98
// MB), 32.4 against 32.5 at 28 (115 MB), 33.3 against 34.3 at 32 (131 MB),
// 38.4 against 41.9 at 40, 44.9 against 54.9 at 64; on the 8-sequence fp32
// recipe 30.1 against 30.3 at B = 80 (102 MB), 32.1 against 33.4 at 96 (123
// MB), 34.6 against 37.4 at 112 (143 MB). With 2, 3, 4 pairs in the first
// phase: 46.8, 44.9, 46.2 at B = 64, 72.8, 70.3, 72.6 at 128; 4 ties 3 only
// at B = 24.
constexpr int64_t kTwoPhaseBytes = int64_t(112) << 20;
int32_t auto_phase1_pairs(int64_t B, int32_t gamma, int32_t V, int32_t dtype) {
    // (compared as B V, below 2^62 for int32 shapes, so nothing overflows)
    const int64_t per = 2 * static_cast<int64_t>(gamma) * elem_bytes(dtype);
    return B * static_cast<int64_t>(V) >= ceil_div(kTwoPhaseBytes, per) ? phase1_pairs(gamma) : 0;
}

int compute_units(int dev) {
    auto it = g_cus.find(dev);
    if (it != g_cus.end()) return it->second;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 1;
    g_cus[dev] = n;
    return n;
}

// sync layout: counters, decision words and draw records, the error word
// (256 bytes), the draft sampler's tagged range words
size_t sync_bytes(int64_t cnt_words, int64_t dec_words, int64_t tag_words = 0) {
    return align_up(static_cast<size_t>(cnt_words) * sizeof(uint32_t), 256) +
           static_cast<size_t>(dec_words) * sizeof(uint64_t) + 256 + static_cast<size_t>(tag_words) * sizeof(uint64_t);
}
uint32_t* err_word(const Workspace& ws) {
    return reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws.sync) +
                                       align_up(static_cast<size_t>(ws.cnt_cap) * sizeof(uint32_t), 256) +
                                       static_cast<size_t>(ws.dec_cap) * sizeof(uint64_t));
}
uint64_t* tag_region(const Workspace& ws) {
    return reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws.sync) +
                                       align_up(static_cast<size_t>(ws.cnt_cap) * sizeof(uint32_t), 256) +
                                       static_cast<size_t>(ws.dec_cap) * sizeof(uint64_t) + 256);
}

// Caller holds g_mu. Grows the buffers of (dev, stream) to fit L (a new sync
// buffer is cleared on the stream) and advances the epoch.
int get_workspace(int dev, hipStream_t stream, const Layout& L, Workspace** out) {
    Workspace& ws = g_ws[std::make_pair(dev, static_cast<void*>(stream))];
    const bool grow_data = ws.bytes < L.bytes;
    const bool grow_sync = ws.cnt_cap < L.cnt_words || ws.dec_cap < L.dec_words || ws.tag_cap < L.tag_words;
    if ((grow_data && ws.data) || (grow_sync && ws.sync))
        if (hipStreamSynchronize(stream) != hipSuccess) return fail(SPEC_EHIP, "hipStreamSynchronize failed");
    if (grow_data) {
        if (ws.data) (void)hipFree(ws.data);
        ws.data = nullptr;
        ws.bytes = 0;
        const size_t want = align_up(L.bytes + L.bytes / 4, 1 << 20);
        if (hipMalloc(&ws.data, want) != hipSuccess) {
            ws.data = nullptr;
            (void)hipGetLastError();
            return fail(SPEC_ENOMEM, "hipMalloc of the workspace failed");
        }
        ws.bytes = want;
    }
    if (grow_sync) {
        if (ws.sync) (void)hipFree(ws.sync);
        ws.sync = nullptr;
        // (keeps what earlier calls needed: the buffer serves every entry point)
        const int64_t cw = std::max<int64_t>(std::max(L.cnt_words + L.cnt_words / 4, ws.cnt_cap), 1024);
        const int64_t dw = std::max<int64_t>(std::max(L.dec_words + L.dec_words / 4, ws.dec_cap), 1024);
        const int64_t tw = std::max<int64_t>(L.tag_words + L.tag_words / 4, ws.tag_cap);
        ws.cnt_cap = ws.dec_cap = ws.tag_cap = 0;
        const size_t sb = sync_bytes(cw, dw, tw);
        if (hipMalloc(reinterpret_cast<void**>(&ws.sync), sb) != hipSuccess) {
            ws.sync = nullptr;
            (void)hipGetLastError();
            return fail(SPEC_ENOMEM, "hipMalloc of the workspace failed");
        }
        if (hipMemsetAsync(ws.sync, 0, sb, stream) != hipSuccess) {
            (void)hipFree(ws.sync);
            ws.sync = nullptr;
            return fail(SPEC_EHIP, "hipMemsetAsync of the workspace failed");
        }
        ws.cnt_cap = cw;
        ws.dec_cap = dw;
        ws.tag_cap = tw;
        ws.epoch = 0;
    }
    if (++ws.epoch == 0) {
        // 2^32 calls on this workspace: clear the tagged words before the tag repeats
        char* dec = reinterpret_cast<char*>(ws.sync) + align_up(static_cast<size_t>(ws.cnt_cap) * sizeof(uint32_t), 256);
        if (hipMemsetAsync(dec, 0, static_cast<size_t>(ws.dec_cap) * sizeof(uint64_t), stream) != hipSuccess)
            return fail(SPEC_EHIP, "hipMemsetAsync of the workspace failed");
        if (ws.tag_cap > 0 &&
            hipMemsetAsync(tag_region(ws), 0, static_cast<size_t>(ws.tag_cap) * sizeof(uint64_t), stream) != hipSuccess)
            return fail(SPEC_EHIP, "hipMemsetAsync of the workspace failed");
        ws.epoch = 1;
    }
    *out = &ws;
    return SPEC_OK;
}

// --------------------------------------------------------------------------
// The scratch of spec_verify_noalloc: a fixed device array (one copy per GPU
// the library runs on, held until the process ends) that stands in for the
// allocated workspace: partial slots and residual masses first, then the
// counters, the group void words and the error word. Host code never passes
// the array's name to a kernel (on the host it is a stand-in, not a device
// address): the address comes from hipGetSymbolAddress, once per device.
// --------------------------------------------------------------------------
constexpr size_t kScratchData = size_t(8) << 20;        // partial slots and residual masses
constexpr int64_t kScratchCntWords = int64_t(128) << 10;  // counters (two per group, kSyncStride words apart)
constexpr int64_t kScratchDecWords = int64_t(16) << 10;   // group void words (64-bit)
constexpr size_t kScratchSync = size_t(kScratchCntWords) * sizeof(uint32_t) +
                                size_t(kScratchDecWords) * sizeof(uint64_t) + 256;
constexpr size_t kScratchBytes = kScratchData + kScratchSync;

}  // namespace
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
namespace {

std::map<int, unsigned char*> g_scratch;  // device -> device address of `scratch` (under g_mu)

__global__ void k_zero_words(uint32_t* p, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = 0u;
}

// Caller holds g_mu. The device address of this device's scratch; the first
// call on a device looks it up and clears its counter, void and error words
// on `stream` (with a kernel, so that a capturing caller records no memset).
int scratch_workspace(int dev, hipStream_t stream, Workspace* out) {
    auto it = g_scratch.find(dev);
    unsigned char* base = nullptr;
    if (it != g_scratch.end()) {
        base = it->second;
    } else {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return fail(SPEC_EHIP, "hipGetSymbolAddress of the scratch array failed");
        }
        base = static_cast<unsigned char*>(ptr);
        const int64_t words = static_cast<int64_t>(kScratchSync / sizeof(uint32_t));
        hipLaunchKernelGGL(k_zero_words, dim3(256), dim3(256), 0, stream,
                           reinterpret_cast<uint32_t*>(base + kScratchData), words);
        if (hipGetLastError() != hipSuccess) return fail(SPEC_EHIP, "clearing the scratch array failed");
        g_scratch[dev] = base;
    }
    Workspace ws;
    ws.data = base;
    ws.bytes = kScratchData;
    ws.sync = reinterpret_cast<uint32_t*>(base + kScratchData);
    ws.cnt_cap = kScratchCntWords;
    ws.dec_cap = kScratchDecWords;
    ws.tag_cap = 0;
    ws.epoch = 1;  // the group-major order's words are reset by their last user, not told apart by epoch
    *out = ws;
    return SPEC_OK;
}

void bind_workspace(Layout& L, const Workspace& ws) {
    char* base = static_cast<char*>(ws.data);
    Params& p = L.p;
    p.part_m = reinterpret_cast<float*>(base + L.off_pm);
    p.part_r = reinterpret_cast<float*>(base + L.off_pr);
    p.part_s = reinterpret_cast<double*>(base + L.off_ps);
    p.part_i = reinterpret_cast<int32_t*>(base + L.off_pi);
    p.tok_l = reinterpret_cast<float*>(base + L.off_tok);
    p.msum = reinterpret_cast<double*>(base + L.off_msum);
    p.sub_r = reinterpret_cast<double*>(base + L.off_subr);
    p.sub_R = reinterpret_cast<float*>(base + L.off_subR);
    p.cnt_s = ws.sync;
    p.cnt_r = ws.sync + static_cast<int64_t>(p.B) * kSyncStride;
    char* s = reinterpret_cast<char*>(ws.sync);
    p.cnt = ws.sync;
    const size_t off_dec = align_up(static_cast<size_t>(ws.cnt_cap) * sizeof(uint32_t), 256);
    p.dec = reinterpret_cast<uint64_t*>(s + off_dec);
    p.rec = p.dec + static_cast<int64_t>(p.B) * (p.gamma + 1);
    p.err = err_word(ws);
    p.epoch = ws.epoch;
    p.wait = wait_ticks();
}

// Timing events, when given, are bound to the kernel dispatch itself (its
// start and end timestamps), so they add no packets to the stream.
template <int DT, bool VEC>
void launch_t(int mode, const Layout& L, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    const dim3 grid(static_cast<unsigned>(L.blocks)), block(kBlock);
    if (L.group && mode == kGreedy)
        hipExtLaunchKernelGGL((k_group<DT, VEC, kGreedy>), grid, block, L.lds, st, e0, e1, 0, L.p);
    else if (L.group)
        hipExtLaunchKernelGGL((k_group<DT, VEC, kSample>), grid, block, L.lds, st, e0, e1, 0, L.p);
    else if (mode == kSample)
        hipExtLaunchKernelGGL((k_verify<DT, VEC, kSample>), grid, block, 0, st, e0, e1, 0, L.p);
    else if (mode == kGreedy)
        hipExtLaunchKernelGGL((k_verify<DT, VEC, kGreedy>), grid, block, 0, st, e0, e1, 0, L.p);
    else
        hipExtLaunchKernelGGL((k_verify<DT, VEC, kRows>), grid, block, 0, st, e0, e1, 0, L.p);
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
int check_size(int, const Layout& L) {
    const int64_t chunks = L.units * (L.group ? L.p.rps : 2) * static_cast<int64_t>(L.p.nchunk);
    if (chunks >= (int64_t(1) << 31) || L.blocks < 1 || L.blocks * kBlock >= (int64_t(1) << 32))
        return fail(SPEC_EINVAL, "problem too large");
    return SPEC_OK;
}

// Draft sampler geometry: rows of nw wavefront ranges of kDraftCw chunks,
// four ranges per block, then one closing wavefront per row. The ranges'
// tagged words live in the workspace's tag region (cleared when allocated and
// when the epoch wraps; each call's words carry its own epoch).
struct DraftLayout {
    DraftParams d;
    int64_t blocks;
    Layout ws;  // the sizes the workspace must hold
};

DraftLayout plan_draft(int64_t rows, int32_t V, int32_t dtype, bool vec) {
    DraftLayout L{};
    DraftParams& d = L.d;
    d.rows = rows;
    d.V = V;
    d.nchunk = static_cast<int32_t>(ceil_div(V, chunk_elems(dtype, vec)));
    d.nw = static_cast<int32_t>(ceil_div(d.nchunk, kDraftCw));
    d.nbr = static_cast<int32_t>(ceil_div(d.nw, kWavesPerBlock));
    L.blocks = rows * d.nbr + ceil_div(rows, kWavesPerBlock);  // statistics blocks, then closing blocks
    L.ws.bytes = 0;
    L.ws.cnt_words = 0;
    L.ws.dec_words = 0;
    L.ws.tag_words = rows * d.nw * kDraftWords;
    return L;
}

void bind_draft(DraftLayout& L, const Workspace& ws) {
    DraftParams& d = L.d;
    d.part = tag_region(ws);
    d.epoch = ws.epoch;
    d.err = err_word(ws);
    d.wait = wait_ticks();
}

template <int DT, bool VEC>
void launch_draft_t(bool greedy, const DraftLayout& L, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    const dim3 grid(static_cast<unsigned>(L.blocks)), block(kBlock);
    if (greedy) hipExtLaunchKernelGGL((k_draft<DT, VEC, true, false>), grid, block, 0, st, e0, e1, 0, L.d);
    else if (L.d.out_h) hipExtLaunchKernelGGL((k_draft<DT, VEC, false, true>), grid, block, 0, st, e0, e1, 0, L.d);
    else hipExtLaunchKernelGGL((k_draft<DT, VEC, false, false>), grid, block, 0, st, e0, e1, 0, L.d);
}

void launch_draft(int32_t dtype, bool vec, bool greedy, const DraftLayout& L, hipStream_t st, hipEvent_t e0,
                  hipEvent_t e1) {
    if (dtype == SPEC_F32) {
        if (vec) launch_draft_t<SPEC_F32, true>(greedy, L, st, e0, e1);
        else launch_draft_t<SPEC_F32, false>(greedy, L, st, e0, e1);
    } else {
        if (vec) launch_draft_t<SPEC_BF16, true>(greedy, L, st, e0, e1);
        else launch_draft_t<SPEC_BF16, false>(greedy, L, st, e0, e1);
    }
}

template <int DT, bool VEC>
void launch_overlap_t(const Params& P, const OverlapParams& O, int64_t blocks, hipStream_t st, hipEvent_t e0,
                      hipEvent_t e1) {
    hipExtLaunchKernelGGL((k_overlap<DT, VEC>), dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, st, e0, e1, 0,
                          P, O);
}

}  // namespace

// ==========================================================================
// C ABI
// ==========================================================================
extern "C" {

int32_t spec_verify_abi_version(void) { return 6; }

int64_t spec_verify_set_wait_limit(int64_t ticks) {
    return g_wait_limit.exchange(ticks < 0 ? -1 : ticks);
}

int spec_verify_status(void* stream, int32_t* timed_out) {
    if (!timed_out) return fail(SPEC_EINVAL, "null pointer argument");
    *timed_out = 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPEC_EHIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(g_mu);
    Workspace ws;
    auto it = g_ws.find(std::make_pair(dev, stream));
    if (it != g_ws.end() && it->second.sync) {
        ws = it->second;
    } else if (g_scratch.count(dev)) {  // spec_verify_noalloc's scratch on this device
        if (int rc = scratch_workspace(dev, st, &ws)) return rc;
    } else {
        return SPEC_OK;  // nothing ran on this stream
    }
    uint32_t word = 0;
    if (hipMemcpyAsync(&word, err_word(ws), sizeof(word), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return fail(SPEC_EHIP, "reading the workspace's error word failed");
    if (word == 0) return SPEC_OK;
    *timed_out = 1;
    // clear the word, and scrub the counters (a wait whose drain also ran out
    // may have left one behind)
    if (hipMemsetAsync(err_word(ws), 0, sizeof(uint32_t), st) != hipSuccess ||
        hipMemsetAsync(ws.sync, 0, static_cast<size_t>(ws.cnt_cap) * sizeof(uint32_t), st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return fail(SPEC_EHIP, "clearing the workspace's error word failed");
    return SPEC_OK;
}

const char* spec_verify_last_error(void) { return g_last_error.c_str(); }

int32_t spec_verify_schedule(int32_t B, int32_t gamma, int32_t V, int32_t dtype, float temperature) {
    if (B < 1 || gamma < 1 || gamma > SPEC_MAX_GAMMA || V < 1 || (dtype != SPEC_F32 && dtype != SPEC_BF16) ||
        !(temperature >= 0.0f))
        return fail(SPEC_EINVAL, "bad shape, dtype or temperature");
    if (temperature == 0.0f) return SPEC_SCHEDULE_EARLY_STOP;
    if (auto_position_major(B, V, dtype)) return SPEC_SCHEDULE_EARLY_STOP;
    return auto_phase1_pairs(B, gamma, V, dtype) > 0 ? SPEC_SCHEDULE_GROUP_TWO_PHASE : SPEC_SCHEDULE_GROUP;
}

size_t spec_verify_workspace_bytes(int32_t B, int32_t gamma, int32_t V, int32_t dtype, float temperature) {
    if (B < 1 || gamma < 1 || gamma > SPEC_MAX_GAMMA || V < 1 || (dtype != SPEC_F32 && dtype != SPEC_BF16))
        return 0;
    const bool vec = (static_cast<int64_t>(V) * elem_bytes(dtype)) % 16 == 0;
    int dev = 0;
    (void)hipGetDevice(&dev);
    std::lock_guard<std::mutex> lk(g_mu);
    const int cus = compute_units(dev);
    const int mode = temperature == 0.0f ? kGreedy : kSample;
    const Layout Lp = plan(mode, B, gamma, V, dtype, vec, cus);
    // (T == 0: the selectable group-major order; T > 0: with the bonus row
    // deferred, whose layout adds the subsegment references)
    const Layout Lg = plan_group(B, gamma, V, dtype, vec, cus, mode, mode == kSample);
    return std::max(Lp.bytes, Lg.bytes) + sync_bytes(std::max(Lp.cnt_words, Lg.cnt_words), Lp.dec_words);
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
    const int mode = greedy ? kGreedy : kSample;
    const int32_t sched = extras ? extras->schedule : SPEC_SCHEDULE_AUTO;
    if (sched < SPEC_SCHEDULE_AUTO || sched > SPEC_SCHEDULE_GROUP_TWO_PHASE)
        return fail(SPEC_EINVAL, "extras->schedule must be one of the spec_schedule_t values");
    const bool per_row = extras && (extras->row_max || extras->row_sumexp || extras->p_draft || extras->q_draft ||
                                    extras->argmax);
    // group-major at T > 0: the bonus row is left to the closing blocks of the
    // sequences that accept every draft token, unless per-row values or Z are
    // asked for (they are defined for every row and sequence)
    const bool defer = !greedy && !per_row && !(extras && extras->Z);
    // the size limits do not depend on the device: checked before any HIP call
    if (int rc = check_size(mode, plan(mode, B, gamma, V, dtype, vec, 1))) return rc;
    if (!greedy || sched == SPEC_SCHEDULE_GROUP || sched == SPEC_SCHEDULE_GROUP_TWO_PHASE) {
        if (int rc = check_size(mode, plan_group(B, gamma, V, dtype, vec, 1, mode, defer, phase1_pairs(gamma))))
            return rc;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPEC_EHIP, "hipGetDevice failed");

    std::lock_guard<std::mutex> lk(g_mu);
    const int cus = compute_units(dev);
    Layout L = plan(mode, B, gamma, V, dtype, vec, cus);
    bool early = true;
    if (greedy && (sched == SPEC_SCHEDULE_GROUP || sched == SPEC_SCHEDULE_GROUP_TWO_PHASE)) {
        L = plan_group(B, gamma, V, dtype, vec, cus, kGreedy);
    } else if (!greedy) {
        // auto: position-major with the early stop once one position's row
        // pairs are long enough, else group-major (in two phases where its
        // rows are)
        const bool group = sched == SPEC_SCHEDULE_AUTO ? !auto_position_major(B, V, dtype)
                                                       : sched == SPEC_SCHEDULE_GROUP || sched == SPEC_SCHEDULE_GROUP_TWO_PHASE;
        const int32_t p0 = sched == SPEC_SCHEDULE_AUTO ? auto_phase1_pairs(B, gamma, V, dtype)
                                                       : (sched == SPEC_SCHEDULE_GROUP_TWO_PHASE ? phase1_pairs(gamma) : 0);
        if (group) L = plan_group(B, gamma, V, dtype, vec, cus, kSample, defer, p0);
        early = sched != SPEC_SCHEDULE_POSITION;
    }
    Workspace* ws = nullptr;
    if (int rc = get_workspace(dev, st, L, &ws)) return rc;
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
    // per-row values are wanted for every row: then every row is read
    p.skip = early && !per_row ? 1 : 0;
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

int spec_verify_noalloc(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                        int32_t B, int32_t gamma, int32_t V, int32_t dtype, float temperature, uint64_t seed,
                        int32_t* out_tokens, int32_t* out_n_accepted, void* stream) {
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
    const int mode = greedy ? kGreedy : kSample;
    if (int rc = check_size(mode, plan_group(B, gamma, V, dtype, vec, 1, mode, !greedy))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPEC_EHIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(g_mu);
    // always the group-major order: its counters are reset by their last user
    // and nothing on its normal path is told apart by the call's epoch
    Layout L = plan_group(B, gamma, V, dtype, vec, compute_units(dev), mode, !greedy);
    if (L.bytes > kScratchData || L.cnt_words > kScratchCntWords || L.dec_words > kScratchDecWords)
        return fail(SPEC_EINVAL, "problem exceeds the no-alloc scratch (at most 1024 sequences and 8 MiB of "
                                 "partial slots and residual masses)");
    Workspace ws;
    if (int rc = scratch_workspace(dev, st, &ws)) return rc;
    bind_workspace(L, ws);
    Params& p = L.p;
    p.c32 = c32;
    p.seed = seed;
    p.b_offset = 0;
    p.tgt = target_logits;
    p.dft = greedy ? nullptr : draft_logits;
    p.tokens = draft_tokens;
    p.out_tokens = out_tokens;
    p.out_n = out_n_accepted;
    p.skip = 0;
    launch(dtype, vec, mode, L, st);
    return check_launch("verification kernel");
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
    if (int rc = check_size(kRows, plan(kRows, rows, 1, V, dtype, vec, 1))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPEC_EHIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(g_mu);
    Layout L = plan(kRows, rows, 1, V, dtype, vec, compute_units(dev));
    Workspace* ws = nullptr;
    if (int rc = get_workspace(dev, st, L, &ws)) return rc;
    bind_workspace(L, *ws);
    L.p.c32 = c32;
    L.p.tgt = logits;
    L.p.rows_max = row_max;
    L.p.rows_sumexp = row_sumexp;
    launch(dtype, vec, kRows, L, st);
    return check_launch("statistics kernel");
}

int spec_draft_sample_ex(const void* logits, int32_t B, int32_t n, int32_t V, int32_t dtype, float temperature,
                         uint64_t seed, int64_t pos0, int64_t b_offset, int32_t* out_tokens, double* out_q,
                         void* stream, const spec_draft_extras_t* extras) {
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return fail(SPEC_EDTYPE, "dtype must be SPEC_F32 or SPEC_BF16");
    if (B < 1 || n < 1 || V < 1) return fail(SPEC_EINVAL, "B, n and V must be >= 1");
    if (pos0 < 0 || b_offset < 0) return fail(SPEC_EINVAL, "pos0 and b_offset must be >= 0");
    if (!(temperature >= 0.0f)) return fail(SPEC_EINVAL, "temperature must be >= 0 and not NaN");
    if (!logits || !out_tokens) return fail(SPEC_EINVAL, "null pointer argument");
    const bool greedy = temperature == 0.0f;
    const float c32 = greedy ? 0.0f : fold_temperature(temperature);
    if (!greedy && !(std::isfinite(c32) && c32 > 0.0f))
        return fail(SPEC_EINVAL, "temperature too small or too large for fp32 exponent scaling");
    const int64_t rows = static_cast<int64_t>(B) * n;
    const bool vec = (static_cast<int64_t>(V) * elem_bytes(dtype)) % 16 == 0 && aligned16(logits);
    DraftLayout L = plan_draft(rows, V, dtype, vec);

    if (rows >= (int64_t(1) << 31) || L.blocks * kBlock >= (int64_t(1) << 32))
        return fail(SPEC_EINVAL, "problem too large");
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPEC_EHIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(g_mu);
    Workspace* ws = nullptr;
    if (int rc = get_workspace(dev, st, L.ws, &ws)) return rc;
    bind_draft(L, *ws);
    DraftParams& d = L.d;
    d.logits = logits;
    d.n = n;
    d.c32 = c32;
    d.seed = seed;
    d.pos0 = pos0;
    d.b_offset = b_offset;
    d.out_tokens = out_tokens;
    d.out_q = out_q;
    d.out_h = extras ? extras->entropy : nullptr;
    hipEvent_t e0 = extras ? static_cast<hipEvent_t>(extras->events[0]) : nullptr;
    hipEvent_t e1 = extras ? static_cast<hipEvent_t>(extras->events[1]) : nullptr;
    launch_draft(dtype, vec, greedy, L, st, e0, e1);
    return check_launch("draft sampling kernel");
}

int spec_expected_accept(const void* target_logits, const void* draft_logits, int32_t B, int32_t gamma, int32_t V,
                         int32_t dtype, float temperature, double* out_beta, void* stream) {
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return fail(SPEC_EDTYPE, "dtype must be SPEC_F32 or SPEC_BF16");
    if (B < 1 || gamma < 1 || V < 1) return fail(SPEC_EINVAL, "B, gamma and V must be >= 1");
    if (!(temperature > 0.0f)) return fail(SPEC_EINVAL, "temperature must be > 0");
    if (!target_logits || !draft_logits || !out_beta) return fail(SPEC_EINVAL, "null pointer argument");
    const float c32 = fold_temperature(temperature);
    if (!(std::isfinite(c32) && c32 > 0.0f)) return fail(SPEC_EINVAL, "temperature out of range");
    const int64_t pairs = static_cast<int64_t>(B) * gamma;
    const int64_t trows = static_cast<int64_t>(B) * (gamma + 1);
    if (trows >= (int64_t(1) << 31) || 2 * pairs >= (int64_t(1) << 31)) return fail(SPEC_EINVAL, "problem too large");
    const bool vec = (static_cast<int64_t>(V) * elem_bytes(dtype)) % 16 == 0 && aligned16(target_logits) &&
                     aligned16(draft_logits);
    Layout Ls = plan(kRows, 2 * pairs, 1, V, dtype, vec, 1);
    if (int rc = check_size(kRows, Ls)) return rc;
    const int32_t nchunk = static_cast<int32_t>(ceil_div(V, chunk_elems(dtype, vec)));
    const int32_t nw = static_cast<int32_t>(ceil_div(nchunk, kDraftCw));
    const int32_t nbr = static_cast<int32_t>(ceil_div(nw, kWavesPerBlock));
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPEC_EHIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(g_mu);
    const int cus = compute_units(dev);
    // the statistics of each pair's target row (each sequence's bonus row is
    // not read) and draft row, row 2p and 2p + 1
    Ls = plan(kRows, 2 * pairs, 1, V, dtype, vec, cus);
    const int64_t sbp = 2 * static_cast<int64_t>(Ls.p.nb1);
    const int64_t blocks = pairs * (sbp + nbr) + ceil_div(pairs, kWavesPerBlock);
    if (blocks * kBlock >= (int64_t(1) << 32)) return fail(SPEC_EINVAL, "problem too large");
    // data: the statistics blocks' slots, then the row statistics and the
    // overlap partials; sync: the statistics blocks' row counters, the pairs'
    // range counters, then the pairs' finished-row counters (one launch uses
    // all three at once)
    const int64_t srows = 2 * pairs;
    const size_t o_m = align_up(Ls.bytes, 256);
    const size_t o_s = align_up(o_m + static_cast<size_t>(srows) * sizeof(float), 256);
    const size_t o_pt = align_up(o_s + static_cast<size_t>(srows) * sizeof(double), 256);
    const int64_t o_cnt = ceil_div(Ls.cnt_words, kSyncStride) * kSyncStride;
    const int64_t o_done = o_cnt + ceil_div(pairs * kDraftStride, kSyncStride) * kSyncStride;
    Layout need{};
    need.bytes = align_up(o_pt + static_cast<size_t>(pairs) * nw * sizeof(double), 256);
    need.cnt_words = o_done + pairs * kSyncStride;
    need.dec_words = Ls.dec_words;
    Workspace* ws = nullptr;
    if (int rc = get_workspace(dev, st, need, &ws)) return rc;
    char* base = static_cast<char*>(ws->data);
    float* m_all = reinterpret_cast<float*>(base + o_m);
    double* s_all = reinterpret_cast<double*>(base + o_s);
    bind_workspace(Ls, *ws);
    Ls.p.c32 = c32;
    Ls.p.tgt = target_logits;
    Ls.p.dft = draft_logits;
    Ls.p.rows_split = 2 * pairs;
    Ls.p.pair_rows = 1;
    Ls.p.tgt_group = gamma;
    Ls.p.rows_max = m_all;
    Ls.p.rows_sumexp = s_all;
    Ls.p.tree_done = ws->sync + o_done;  // each row counts in at its pair
    Ls.p.tree_n = 2;
    OverlapParams O{};
    O.tgt = target_logits;
    O.dft = draft_logits;
    O.B = B;
    O.gamma = gamma;
    O.V = V;
    O.nchunk = nchunk;
    O.nw = nw;
    O.nbr = nbr;
    O.c32 = c32;
    O.m_t = m_all;
    O.s_t = s_all;
    O.part = reinterpret_cast<double*>(base + o_pt);
    O.cnt = ws->sync + o_cnt;
    O.err = Ls.p.err;
    O.out_beta = out_beta;
    O.sbp = sbp;
    O.lag = std::min<int64_t>(pairs, kOverlapLag);
    O.rows_done = Ls.p.tree_done;
    O.wait = Ls.p.wait;
    if (dtype == SPEC_F32) {
        if (vec) launch_overlap_t<SPEC_F32, true>(Ls.p, O, blocks, st, nullptr, nullptr);
        else launch_overlap_t<SPEC_F32, false>(Ls.p, O, blocks, st, nullptr, nullptr);
    } else {
        if (vec) launch_overlap_t<SPEC_BF16, true>(Ls.p, O, blocks, st, nullptr, nullptr);
        else launch_overlap_t<SPEC_BF16, false>(Ls.p, O, blocks, st, nullptr, nullptr);
    }
    return check_launch("expected acceptance kernel");
}

int spec_tree_verify(const void* target_logits, const void* draft_logits, const int32_t* parent,
                     const int32_t* token, int32_t B, int32_t N, int32_t V, int32_t dtype, float temperature,
                     float threshold, int32_t* out_tokens, int32_t* out_nodes, int32_t* out_n, void* stream) {
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return fail(SPEC_EDTYPE, "dtype must be SPEC_F32 or SPEC_BF16");
    if (B < 1 || N < 2 || V < 1) return fail(SPEC_EINVAL, "need B >= 1, N >= 2 and V >= 1");
    if (!(temperature >= 0.0f)) return fail(SPEC_EINVAL, "temperature must be >= 0 and not NaN");
    if (std::isnan(threshold)) return fail(SPEC_EINVAL, "threshold must not be NaN");
    const bool greedy = temperature == 0.0f;
    if (!target_logits || !parent || !token || !out_tokens || !out_n || (!greedy && !draft_logits))
        return fail(SPEC_EINVAL, "null pointer argument");
    const float c32 = greedy ? 0.0f : fold_temperature(temperature);
    if (!greedy && !(std::isfinite(c32) && c32 > 0.0f)) return fail(SPEC_EINVAL, "temperature out of range");
    const int64_t rows = static_cast<int64_t>(B) * N;
    if (rows >= (int64_t(1) << 31)) return fail(SPEC_EINVAL, "problem too large");
    const bool vec = (static_cast<int64_t>(V) * elem_bytes(dtype)) % 16 == 0 && aligned16(target_logits) &&
                     (greedy || aligned16(draft_logits));
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPEC_EHIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(g_mu);
    const int cus = compute_units(dev);
    TreeParams Q{};
    Q.tgt = target_logits;
    Q.dft = greedy ? nullptr : draft_logits;
    Q.parent = parent;
    Q.token = token;
    Q.B = B;
    Q.N = N;
    Q.V = V;
    Q.T = greedy ? 0.0 : static_cast<double>(temperature);
    Q.threshold = threshold;
    Q.out_tokens = out_tokens;
    Q.out_nodes = out_nodes;
    Q.out_n = out_n;
    const bool hold = N <= kTreeHold * kWave;
    const dim3 grid(static_cast<unsigned>(ceil_div(B, kWavesPerBlock))), block(kBlock);
    // every node's row statistics (T > 0: both models; T == 0: the target
    // argmax) in front of the walk; the statistics kernels use the front of
    // the workspace, the per-row results follow. At T > 0 a tree that the walk
    // holds whole is walked by closing wavefronts of the statistics launch.
    if (!greedy) {
        if (2 * rows >= (int64_t(1) << 31)) return fail(SPEC_EINVAL, "problem too large");
        Layout L = plan(kRows, 2 * rows, 1, V, dtype, vec, cus);  // target rows, then draft rows
        if (int rc = check_size(kRows, L)) return rc;
        const int64_t tree_blocks = ceil_div(B, kWavesPerBlock);
        if ((L.blocks + tree_blocks) * kBlock >= (int64_t(1) << 32)) return fail(SPEC_EINVAL, "problem too large");
        const size_t o_m = align_up(L.bytes, 256);
        const size_t o_s = align_up(o_m + static_cast<size_t>(2 * rows) * sizeof(float), 256);
        Layout need = L;
        need.bytes = align_up(o_s + static_cast<size_t>(2 * rows) * sizeof(double), 256);
        const int64_t o_tree = ceil_div(L.cnt_words, kSyncStride) * kSyncStride;  // the trees' row counters
        if (hold) need.cnt_words = o_tree + static_cast<int64_t>(B) * kSyncStride;
        Workspace* ws = nullptr;
        if (int rc = get_workspace(dev, st, need, &ws)) return rc;
        char* base = static_cast<char*>(ws->data);
        float* m_all = reinterpret_cast<float*>(base + o_m);
        double* s_all = reinterpret_cast<double*>(base + o_s);
        bind_workspace(L, *ws);
        L.p.c32 = c32;
        L.p.tgt = target_logits;
        L.p.dft = draft_logits;
        L.p.rows_split = rows;
        L.p.rows_max = m_all;
        L.p.rows_sumexp = s_all;
        Q.m_t = m_all;
        Q.s_t = s_all;
        Q.m_d = m_all + rows;
        Q.s_d = s_all + rows;
        if (hold) {
            L.p.tree_done = ws->sync + o_tree;
            L.p.tree_n = N;
            Q.first_block = L.blocks;
            Q.done = L.p.tree_done;
            Q.err = L.p.err;
            Q.wait = L.p.wait;
            const dim3 g2(static_cast<unsigned>(L.blocks + tree_blocks));
            if (dtype == SPEC_F32) {
                if (vec) hipLaunchKernelGGL((k_tree<SPEC_F32, true>), g2, block, 0, st, L.p, Q);
                else hipLaunchKernelGGL((k_tree<SPEC_F32, false>), g2, block, 0, st, L.p, Q);
            } else {
                if (vec) hipLaunchKernelGGL((k_tree<SPEC_BF16, true>), g2, block, 0, st, L.p, Q);
                else hipLaunchKernelGGL((k_tree<SPEC_BF16, false>), g2, block, 0, st, L.p, Q);
            }
            return check_launch("tree kernel");
        }
        launch(dtype, vec, kRows, L, st);
        if (int rc = check_launch("statistics kernel")) return rc;
    } else {
        DraftLayout L = plan_draft(rows, V, dtype, vec);
        if (L.blocks * kBlock >= (int64_t(1) << 32)) return fail(SPEC_EINVAL, "problem too large");
        const size_t o_am = align_up(L.ws.bytes, 256);
        Layout need = L.ws;
        need.bytes = align_up(o_am + static_cast<size_t>(rows) * sizeof(int32_t), 256);
        Workspace* ws = nullptr;
        if (int rc = get_workspace(dev, st, need, &ws)) return rc;
        bind_draft(L, *ws);
        int32_t* am = reinterpret_cast<int32_t*>(static_cast<char*>(ws->data) + o_am);
        L.d.logits = target_logits;
        L.d.n = 1;
        L.d.c32 = 0.0f;
        L.d.out_tokens = am;
        L.d.out_q = nullptr;
        L.d.out_h = nullptr;
        launch_draft(dtype, vec, true, L, st, nullptr, nullptr);
        if (int rc = check_launch("argmax kernel")) return rc;
        Q.amax = am;
    }
    if (dtype == SPEC_F32) {
        if (hold) hipLaunchKernelGGL((k_tree_walk<SPEC_F32, true>), grid, block, 0, st, Q);
        else hipLaunchKernelGGL((k_tree_walk<SPEC_F32, false>), grid, block, 0, st, Q);
    } else {
        if (hold) hipLaunchKernelGGL((k_tree_walk<SPEC_BF16, true>), grid, block, 0, st, Q);
        else hipLaunchKernelGGL((k_tree_walk<SPEC_BF16, false>), grid, block, 0, st, Q);
    }
    return check_launch("tree walk kernel");
}

int spec_draft_sample(const void* logits, int32_t B, int32_t n, int32_t V, int32_t dtype, float temperature,
                      uint64_t seed, int64_t pos0, int64_t b_offset, int32_t* out_tokens, double* out_q,
                      void* stream) {
    return spec_draft_sample_ex(logits, B, n, V, dtype, temperature, seed, pos0, b_offset, out_tokens, out_q,
                                stream, nullptr);
}

}  // extern "C"
