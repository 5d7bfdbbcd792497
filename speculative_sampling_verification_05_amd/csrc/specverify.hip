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
// Three stream-ordered kernels per call (two at T == 0); no kernel waits on
// another work-group and none hands work over through atomics:
//  k_stats         one streaming pass over every target and draft row (all
//                  the compulsory bytes). Each wavefront owns a contiguous
//                  range of 1 KiB chunks of the concatenated rows, keeps per
//                  lane an online max and a sum of 2^(x*c - R) (R an integer
//                  reference, c = log2(e)/T), software-pipelines its 16-byte
//                  loads, and flushes one partial per row piece with wave
//                  reductions. At T == 0 it tracks the argmax (first index of
//                  the maximum) instead.
//  k_accept_resid  a few blocks per sequence. Each block folds the sequence's
//                  partials (one wavefront per row) and repeats the accept
//                  step: lane i takes the two logits of draft token i
//                  (gathered by k_stats), forms alpha in fp64, draws its
//                  Philox uniform, and a ballot finds the first rejection k.
//                  Block 0 writes the accepted tokens and k. Then every
//                  wavefront sums, in fp64, the residual max(0, p - q) of row
//                  k (or p of the bonus row) over 1024-element subsegments.
//                  (k_accept_greedy is its T == 0 counterpart: argmax merge and
//                  accept only.)
//  k_draw          one wavefront per sequence: wave scans of the subsegment
//                  sums give Z and the subsegment holding u*Z; a scan over its
//                  1024 elements, held in registers, gives the first index
//                  whose cumulative mass exceeds u*Z.
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

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kUnroll = SPECVERIFY_STATS_UNROLL;          // chunks per pipelined load group
constexpr int kChunksPerWave = SPECVERIFY_CHUNKS_PER_WAVE; // 1 KiB chunks per stats wavefront
constexpr float kRUnset = -1.0e30f;                       // lane reference before the first finite value
constexpr int kSub = kWave * 16;  // elements per residual subsegment (one wavefront, 16 per lane)
#ifndef SPECVERIFY_TAIL_BLOCK
#define SPECVERIFY_TAIL_BLOCK 512
#endif
constexpr int kTailBlock = SPECVERIFY_TAIL_BLOCK;  // threads per accept/residual block
constexpr int kMaxStage = 2048;                    // partials staged in LDS per sequence (20 bytes each)
constexpr int kMergeBatch = 2;                     // staged partial loads in flight per thread

enum : int { kAcc = 0, kRej = 1, kBad = 2 };

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
__device__ inline double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// --------------------------------------------------------------------------
// Geometry of the statistics pass: rows [0, rows_t) are target rows in memory
// order, rows [rows_t, rows) draft rows (absent at T == 0 and for the
// stand-alone row statistics); each row is nchunk chunks; wave w owns chunks
// [w*cpw, (w+1)*cpw) of the concatenation; row r's partials sit at
// r*maxp + (w - first wave of r).
// --------------------------------------------------------------------------
struct Geom {
    int64_t rows_t;
    int64_t rows;
    int32_t V;
    int32_t nchunk;
    int64_t cpw;
    int64_t nwaves;
    int32_t maxp;
    int32_t gamma;
    const int32_t* tokens;  // draft tokens, or nullptr (no logit gather)
};

template <int DT>
__device__ inline const char* row_ptr(const void* tgt, const void* dft, const Geom& g, int64_t r) {
    return r < g.rows_t ? row_at<DT>(tgt, r * g.V) : row_at<DT>(dft, (r - g.rows_t) * g.V);
}


struct StatsArgs {
    float c32;
    float* part_m;    // max of the piece
    float* part_r;    // integer reference of the piece (T > 0)
    double* part_s;   // sum of 2^(x*c - reference) (T > 0)
    int32_t* part_i;  // first index of the maximum (T == 0)
    float* gath;      // per row: the logit at the row's draft token (written by the piece holding it)
};

// --------------------------------------------------------------------------
// k_stats. State at T > 0: per lane m = max seen and S = sum of
// 2^(fl(x*c - R)) in fp64 (fp32 per load group); R is one integer reference
// for the whole wavefront (kRUnset until the first finite value), set from the
// wave's first group max. A group's exponentials use the current R while its
// max is formed; only if some lane's group max exceeds R + 1 (a ballot) does
// the wave move R up to ceil(wave max * c), rescale S exactly with ldexp and
// redo the group. The flush is then a plain wave sum: every lane shares R.
// --------------------------------------------------------------------------
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

// The logit at index tok, if the load group starting at chunk c0 holds it
// (tok < c_end*CH keeps padding chunks of other pieces out): the lane that
// holds it selects the word from its registers.
template <int DT, bool VEC, int N>
__device__ inline void pick_token(const typename Chunk<DT, VEC>::Raw* raw, int64_t c0, int64_t c_end, int lane,
                                  int64_t tok, float& val, bool& found) {
    using C = Chunk<DT, VEC>;
    const int64_t off = tok - c0 * C::CH;
    if (off >= 0 && off < N * C::CH && tok < c_end * C::CH) {  // wave-uniform, once per row
        const int u = static_cast<int>(off / C::CH);
        const int in = static_cast<int>(off - static_cast<int64_t>(u) * C::CH);
        const int holder = VEC ? in / C::EPL : in % kWave;
        const int v = VEC ? in % C::EPL : in / kWave;
        // word index of the element within the lane's N loads, then a select chain
        const int word = VEC ? u * 4 + (DT == SPEC_F32 ? v : v >> 1) : u * 4 + v;
        uint32_t bits = 0u;
#pragma unroll
        for (int k = 0; k < N; ++k) {
            uint32_t b4[4];
            if constexpr (VEC) {
                b4[0] = raw[k].x; b4[1] = raw[k].y; b4[2] = raw[k].z; b4[3] = raw[k].w;
            } else {
                b4[0] = __float_as_uint(raw[k].x); b4[1] = __float_as_uint(raw[k].y);
                b4[2] = __float_as_uint(raw[k].z); b4[3] = __float_as_uint(raw[k].w);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) bits = word == k * 4 + q ? b4[q] : bits;
        }
        const float x = (!VEC || DT == SPEC_F32) ? __uint_as_float(bits)
                                                 : __uint_as_float((v & 1) ? (bits & 0xFFFF0000u) : (bits << 16));
        if (lane == holder) {
            val = x;
            found = true;
        }
    }
}

template <int DT, bool VEC, bool GREEDY, bool GATHER>
__global__ __launch_bounds__(kBlock) void k_stats(const void* __restrict__ tgt, const void* __restrict__ dft,
                                                  Geom g, StatsArgs sa) {
    using C = Chunk<DT, VEC>;
    using Raw = typename C::Raw;
    using Lane = typename std::conditional<GREEDY, ArgLane, SoftLane>::type;
    const int lane = threadIdx.x & (kWave - 1);
    // wave-uniform bookkeeping in 32-bit scalar registers (the host keeps the
    // chunk count below 2^31): one division per wave finds the first row
    const uint32_t w = blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (w >= static_cast<uint32_t>(g.nwaves)) return;
    const float c = sa.c32;
    const uint32_t nchunk = static_cast<uint32_t>(g.nchunk), cpw = static_cast<uint32_t>(g.cpw);
    const uint32_t total = static_cast<uint32_t>(g.rows) * nchunk;
    uint32_t cc = w * cpw;
    const uint32_t c_end = cc + cpw < total ? cc + cpw : total;
    uint32_t r = cc / nchunk;
    uint32_t first = r * nchunk;
    int32_t k = static_cast<int32_t>(w - first / cpw);  // partial slot of this wave's first piece
    const uint32_t nt_row = static_cast<uint32_t>(g.gamma) + 1u;
    while (cc < c_end) {
        const uint32_t ce = first + nchunk < c_end ? first + nchunk : c_end;
        const char* row = row_ptr<DT>(tgt, dft, g, r);
        const int64_t c0 = cc - first, c1 = ce - first;  // this piece: chunks [c0, c1) of row r
        // the draft token this row scores (T > 0), picked from registers as its
        // chunk streams by
        // (branch-free, and nothing reads the loaded value before tok_ready():
        // the bonus row loads token 0 and has_tok drops it)
        int32_t tok = -1;
        bool has_tok = false;
        if constexpr (GATHER) {
            // index into draft_tokens of the token row r scores (none: the bonus row)
            uint32_t tix;
            if (r >= static_cast<uint32_t>(g.rows_t)) {
                tix = r - static_cast<uint32_t>(g.rows_t);
                has_tok = true;
            } else {
                const uint32_t b = r / nt_row, i = r - b * nt_row;
                tix = b * (nt_row - 1u) + i;
                has_tok = i + 1u < nt_row;
            }
            tok = g.tokens[has_tok ? tix : 0u];
        }
        float tok_logit = 0.0f;
        bool tok_found = false;
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
            for (int u = 0; u < kUnroll; ++u) q[u] = C::load_clamped(row, c0 + gi * kUnroll + u, c_last, lane, g.V);
            __builtin_amdgcn_sched_barrier(0);
        };
        // the token is first needed once the first group is in flight: nothing
        // that reads it may be placed before those loads
        auto tok_ready = [&]() {
            if constexpr (GATHER) asm volatile("" : "+v"(tok) : : "memory");
        };
        auto eat = [&](const Raw* q, int64_t gi) {
            const int64_t cg = c0 + gi * kUnroll;
            consume_group<DT, VEC, kUnroll>(st, q, cg, lane, c);
            if constexpr (GATHER) {
                if (has_tok) pick_token<DT, VEC, kUnroll>(q, cg, c1, lane, tok, tok_logit, tok_found);
            }
        };
        auto eat_last = [&](Raw* q, int64_t gi) {
            const int64_t cg = c0 + gi * kUnroll;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) q[u] = C::mask(q[u], cg + u, c_last, lane, g.V);
            eat(q, gi);
        };
        if (ng == 1) {
            load_last(qa, 0);
            tok_ready();
            eat_last(qa, 0);
        } else {
            load(qa, 0);
            tok_ready();
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
        const int64_t slot = static_cast<int64_t>(r) * g.maxp + k;
        // the wave that ends the row also neutralises the row's unused slots
        // (a row spans maxp - 1 or maxp waves), so merges read every slot
        const bool pad = ce == first + nchunk && lane > 0 && k + lane < g.maxp;
        if constexpr (GREEDY) {
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {  // (value desc, index asc) across the wave
                const float ob = __shfl_xor(st.best, o, kWave);
                const int32_t oa = __shfl_xor(st.at, o, kWave);
                if (ob > st.best || (ob == st.best && oa < st.at)) { st.best = ob; st.at = oa; }
            }
            const bool any_nan = __ballot(st.nan) != 0;
            if (lane == 0) {
                sa.part_m[slot] = any_nan ? NAN : st.best;
                sa.part_i[slot] = st.at;
            } else if (pad) {
                sa.part_m[slot + lane] = -INFINITY;
                sa.part_i[slot + lane] = INT32_MAX;
            }
        } else {
            const float M = wave_max(st.m);
            const float Rw = st.R;  // shared by the wave
            const double Sw = wave_sum(st.S);
            if (lane == 0) {
                sa.part_m[slot] = M;
                sa.part_r[slot] = Rw;
                sa.part_s[slot] = Sw;
            } else if (pad) {
                sa.part_m[slot + lane] = -INFINITY;
                sa.part_r[slot + lane] = kRUnset;
                sa.part_s[slot + lane] = 0.0;
            }
            if (tok_found) sa.gath[r] = tok_logit;
        }
        cc = ce;
        ++r;  // a later piece of this wave starts its row: slot 0
        first += nchunk;
        k = 0;
    }
}

// --------------------------------------------------------------------------
// Merging partials. A row's partials (M_p, R_p, S_p) combine exactly with
// ldexp onto the largest reference R; the result is rebased once to the row
// max: S * 2^(R - M*c), the exponent formed exactly in fp64. The argmax
// partials combine as (value desc, index asc); any NaN marks the row. A row
// has maxp partial slots; the statistics pass fills the one it may leave
// unused with a neutral entry, so every slot can be read blindly.
// --------------------------------------------------------------------------
struct RowStat {
    float m;
    int32_t arg;
    double s;
};

__device__ inline bool usable(float M, double S) { return isfinite(M) && isfinite(S) && S > 0.0; }

// Row j of sequence b as the accept step sees it: target rows 0..gamma first,
// then (T > 0) draft rows 0..gamma-1.
__device__ inline int64_t seq_row(const Geom& g, int64_t b, int j) {
    const int nt = g.gamma + 1;
    return j < nt ? b * nt + j : g.rows_t + b * g.gamma + (j - nt);
}

// One wavefront folds one row: lane k takes slots k, k+64, ...; the lanes
// then combine with butterfly reductions. Every lane returns the row's stats.
template <bool GREEDY>
__device__ inline RowStat fold_row_wave(const Geom& g, const StatsArgs& sa, int64_t r, int lane) {
    const int64_t base = r * g.maxp;
    RowStat o;
    if constexpr (GREEDY) {
        float best = -INFINITY;
        int32_t arg = INT32_MAX;
        bool nan = false;
        for (int k = lane; k < g.maxp; k += kWave) {
            const float v = sa.part_m[base + k];
            const int32_t a = sa.part_i[base + k];
            nan |= (v != v);
            if (v > best || (v == best && a < arg)) { best = v; arg = a; }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ob = __shfl_xor(best, off, kWave);
            const int32_t oa = __shfl_xor(arg, off, kWave);
            if (ob > best || (ob == best && oa < arg)) { best = ob; arg = oa; }
        }
        o.m = __any(nan) ? NAN : best;
        o.arg = arg;
        o.s = 1.0;
    } else {
        float M = -INFINITY, R = kRUnset;
        double S = 0.0;
        for (int k = lane; k < g.maxp; k += kWave) {
            const float mk = sa.part_m[base + k], rk = sa.part_r[base + k];
            const double sk = sa.part_s[base + k];
            const float Rn = fmaxf(R, rk);
            S = rebase(S, R, Rn) + rebase(sk, rk, Rn);
            R = Rn;
            M = fmaxf(M, mk);
        }
        const float Mw = wave_max(M), Rw = wave_max(R);
        const double Sw = wave_sum(rebase(S, R, Rw));
        o.m = Mw;
        o.arg = 0;
        o.s = Sw * exp2(static_cast<double>(Rw) - static_cast<double>(Mw) * static_cast<double>(sa.c32));
    }
    return o;
}

// One thread folds one row from partials staged in LDS (np slots).
template <bool GREEDY>
__device__ inline RowStat fold_row(int np, const float* pm, const float* pr, const double* ps, const int32_t* pi,
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
            if (v > best || (v == best && a < arg)) { best = v; arg = a; }
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

// The nrows rows of sequence b folded into rs[0, nrows) (LDS), by a block of
// NT threads. If their nrows*maxp partials fit the staging buffer (cap
// entries of 20 bytes in dynamic LDS), every thread loads kMergeBatch of them
// at a time, so the merge costs one round trip; then thread j folds row j.
// Otherwise one wavefront folds each row straight from memory.
template <bool GREEDY, int NT>
__device__ inline void merge_seq(const Geom& g, const StatsArgs& sa, int64_t b, int nrows, int cap, char* dyn,
                                 RowStat* rs) {
    const int maxp = g.maxp;
    const int slots = nrows * maxp;
    if (slots <= cap) {
        double* ls = reinterpret_cast<double*>(dyn);
        float* lm = reinterpret_cast<float*>(ls + cap);
        float* lr = lm + cap;
        int32_t* li = reinterpret_cast<int32_t*>(lr + cap);
        for (int t0 = 0; t0 < slots; t0 += kMergeBatch * NT) {
            float vm[kMergeBatch], vr[kMergeBatch];
            double vs[kMergeBatch];
            int32_t vi[kMergeBatch];
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u) {
                const int t = t0 + u * NT + static_cast<int>(threadIdx.x);
                if (t < slots) {
                    const int j = t / maxp;
                    const int64_t at = seq_row(g, b, j) * maxp + (t - j * maxp);
                    vm[u] = sa.part_m[at];
                    if constexpr (GREEDY) {
                        vi[u] = sa.part_i[at];
                    } else {
                        vr[u] = sa.part_r[at];
                        vs[u] = sa.part_s[at];
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u) {
                const int t = t0 + u * NT + static_cast<int>(threadIdx.x);
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
        }
        __syncthreads();
        for (int j = threadIdx.x; j < nrows; j += NT) {
            const int base = j * maxp;
            rs[j] = fold_row<GREEDY>(maxp, lm + base, lr + base, ls + base, li + base, sa.c32);
        }
    } else {
        const int lane = threadIdx.x & (kWave - 1);
        for (int j = threadIdx.x / kWave; j < nrows; j += NT / kWave) {
            const RowStat o = fold_row_wave<GREEDY>(g, sa, seq_row(g, b, j), lane);
            if (lane == 0) rs[j] = o;
        }
    }
    __syncthreads();
}

// What the residual sums and the draw need about the row a sequence resamples
// (see the residual section below for the t units).
struct SeqInfo {
    int32_t k;       // emitted position (0..gamma), -1 = invalid sequence
    float mcp, mcq;  // fl(max*c) of the target row k / draft row k
    int32_t has_q;   // 0 at the bonus row (k == gamma)
    double rho;      // scale_q / scale_p
    double scale_p;  // 2^(mcp - max_p*c) / S_p: probability per t unit
};


struct AcceptArgs {
    const int32_t* tokens;
    const float* gath;  // per row: logit at its draft token (from the statistics pass)
    int32_t B, gamma, V;
    int32_t nsub;       // subsegments per row: ceil(V / kSub)
    int32_t nblk;       // blocks per sequence (T > 0)
    int32_t spb;        // subsegments per block
    int32_t stage;      // partial slots staged in LDS per sequence (0: fold from memory)
    float c32;
    uint64_t seed;
    int64_t b_offset;
    int32_t* out_tokens;
    int32_t* out_n;
    SeqInfo* info;
    double* sub_r;      // [B, nsub] residual mass per subsegment (t units)
    double* sub_p;      // [B, nsub] mass of p per subsegment (t units)
    float* dbg_row_max;
    double* dbg_row_sumexp;
    double* dbg_p;
    double* dbg_q;
    int32_t* dbg_argmax;
};

// --------------------------------------------------------------------------
// Residual in t units. With e_j = 2^(fl(x_j*c - mc)) for the target (p) and
// draft (q) rows, p_j = e_pj * scale_p and q_j = e_qj * scale_q (scale =
// 2^(mc - m*c)/S). Then max(0, p_j - q_j) = scale_p * t_j with
// t_j = max(0, e_pj - rho*e_qj), rho = scale_q/scale_p (one fp64 FMA). The
// inverse-CDF draw is invariant to the common factor; at the bonus row
// t_j = e_pj.
// --------------------------------------------------------------------------
struct ResidRow {
    const char* prow;
    const char* qrow;  // nullptr at the bonus row
    float mcp, mcq;
    double rho;
};

template <int DT>
__device__ inline ResidRow resid_row(const void* tgt, const void* dft, const SeqInfo& s, int64_t b,
                                     int32_t gamma, int32_t V) {
    ResidRow rr;
    rr.prow = row_at<DT>(tgt, (b * (gamma + 1) + s.k) * V);
    rr.qrow = s.has_q ? row_at<DT>(dft, (b * gamma + s.k) * V) : nullptr;
    rr.mcp = s.mcp;
    rr.mcq = s.mcq;
    rr.rho = s.rho;
    return rr;
}

// The residual constants of a row pair from its merged stats (max m, sum S).
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

__device__ inline float t_of_p(float xp, const ResidRow& rr, float c32) {
    return __builtin_amdgcn_exp2f(fmaf(xp, c32, -rr.mcp));
}

__device__ inline double resid_t(double ep, float xq, bool has_q, float c32, const ResidRow& rr) {
    if (!has_q) return ep;
    const double eq = static_cast<double>(__builtin_amdgcn_exp2f(fmaf(xq, c32, -rr.mcq)));
    return fmax(0.0, fma(-eq, rr.rho, ep));
}

// The 16 elements of lane `lane` in subsegment i: j0 = i*kSub + 16*lane, ...
// (p row; q row when has_q). Vector path: 16-byte loads, each taken only if it
// starts below V, which puts it wholly inside the row (V % EPL == 0 there).
// Elements at or beyond V read as -inf in p (no mass).
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
                                : make_uint4(0, 0, 0, 0);
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
            xq[v] = in && has_q ? load_one<DT>(rr.qrow, j0 + v) : 0.0f;
        }
    }
}

// --------------------------------------------------------------------------
// The accept step, run by the first wavefront after merge_seq: lane i takes
// draft token i, forms alpha in fp64, draws its Philox uniform, and a ballot
// finds the first rejection k. Writes the accepted tokens and k (when `emit`),
// and returns the sequence record for the residual.
// --------------------------------------------------------------------------
template <bool GREEDY>
__device__ inline SeqInfo accept_wave(const Geom& g, const AcceptArgs& a, int64_t b, const RowStat* rs, int32_t x,
                                      float lt, float ld, bool emit) {
    const int32_t gamma = a.gamma, V = a.V;
    const int nt = gamma + 1;
    const int i = threadIdx.x;  // lane of wave 0
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
        if (emit && a.dbg_row_max) a.dbg_row_max[b * R + i] = mt;
        if constexpr (GREEDY) {
            amax = t.arg;
            ut = isfinite(mt);
            if (emit && a.dbg_argmax) a.dbg_argmax[b * nt + i] = amax;
        } else {
            st = t.s;
            ut = usable(mt, st);
            if (emit && a.dbg_row_sumexp) a.dbg_row_sumexp[b * R + i] = st;
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
            if (emit && a.dbg_row_max) a.dbg_row_max[b * R + nt + i] = md;
            if (emit && a.dbg_row_sumexp) a.dbg_row_sumexp[b * R + nt + i] = sd;
            double p = NAN, q = NAN;
            if (!ut || !ud || !tok_ok) {
                status = kBad;
            } else {
                const double c = static_cast<double>(a.c32);
                p = exp2((static_cast<double>(lt) - static_cast<double>(mt)) * c) / st;
                q = exp2((static_cast<double>(ld) - static_cast<double>(md)) * c) / sd;
                const double alpha = p == 0.0 ? 0.0 : (q == 0.0 ? 1.0 : fmin(1.0, p / q));
                const double u = philox_uniform(a.seed, static_cast<uint32_t>(b + a.b_offset),
                                                static_cast<uint32_t>(i), 0u);
                status = u < alpha ? kAcc : kRej;
            }
            if (emit && a.dbg_p) a.dbg_p[b * gamma + i] = p;
            if (emit && a.dbg_q) a.dbg_q[b * gamma + i] = q;
        }
    }
    SeqInfo mine{};
    if constexpr (!GREEDY) {
        if (i <= gamma) mine = seq_info(i, i < gamma, mt, st, md, sd, a.c32);
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
            if (!invalid) {
                if (i < k) o = x;
                else if (GREEDY && i == k) o = amax;
            }
            a.out_tokens[b * nt + i] = o;
        }
        if (i == 0) a.out_n[b] = k;
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

// Draft token i and its two logits (gathered by the statistics pass).
template <bool GREEDY>
__device__ inline void load_tokens(const Geom& g, const AcceptArgs& a, int64_t b, int32_t& x, float& lt, float& ld) {
    x = 0;
    lt = 0.0f;
    ld = 0.0f;
    const int i = threadIdx.x;
    if (i < a.gamma) {
        x = a.tokens[b * a.gamma + i];
        if constexpr (!GREEDY) {
            lt = a.gath[b * (a.gamma + 1) + i];
            ld = a.gath[g.rows_t + b * a.gamma + i];
        }
    }
}

// --------------------------------------------------------------------------
// k_accept (T == 0): one block per sequence: argmax merge and the accept step.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_accept_greedy(Geom g, StatsArgs sa, AcceptArgs a) {
    extern __shared__ __align__(16) char dyn[];
    __shared__ RowStat rs[SPEC_MAX_GAMMA + 1];
    const int64_t b = blockIdx.x;
    int32_t x;
    float lt, ld;
    if (threadIdx.x < kWave) load_tokens<true>(g, a, b, x, lt, ld);
    merge_seq<true, kBlock>(g, sa, b, a.gamma + 1, a.stage, dyn, rs);
    if (threadIdx.x < kWave) (void)accept_wave<true>(g, a, b, rs, x, lt, ld, true);
}

// --------------------------------------------------------------------------
// k_accept_resid (T > 0): nblk blocks per sequence. Every block merges the
// sequence's partials and repeats the accept step (a few kilobytes of loads
// and a few hundred instructions); block 0 writes the tokens, k and the
// sequence record. Then each wavefront takes subsegments of row k and writes
// their fp64 residual mass and p mass (t units).
// --------------------------------------------------------------------------
template <int DT, bool VEC>
__global__ __launch_bounds__(kTailBlock) void k_accept_resid(const void* __restrict__ tgt,
                                                             const void* __restrict__ dft, Geom g, StatsArgs sa,
                                                             AcceptArgs a) {
    extern __shared__ __align__(16) char dyn[];
    __shared__ RowStat rs[2 * SPEC_MAX_GAMMA + 1];
    __shared__ SeqInfo shi;
    constexpr int kTailWaves = kTailBlock / kWave;
    const int64_t b = blockIdx.x / a.nblk;
    const int32_t s = static_cast<int32_t>(blockIdx.x - b * a.nblk);
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    int32_t x;
    float lt, ld;
    if (w == 0) load_tokens<false>(g, a, b, x, lt, ld);
    merge_seq<false, kTailBlock>(g, sa, b, 2 * a.gamma + 1, a.stage, dyn, rs);
    if (w == 0) {
        const SeqInfo si = accept_wave<false>(g, a, b, rs, x, lt, ld, s == 0);
        if (lane == 0) {
            shi = si;
            if (s == 0) a.info[b] = si;
        }
    }
    __syncthreads();
    const SeqInfo in = shi;
    if (in.k < 0) return;  // block-uniform
    const float c32 = a.c32;
    const ResidRow rr = resid_row<DT>(tgt, dft, in, b, a.gamma, a.V);
    const bool has_q = rr.qrow != nullptr;
    const int32_t i_end = (s + 1) * a.spb < a.nsub ? (s + 1) * a.spb : a.nsub;
    for (int32_t i = s * a.spb + w; i < i_end; i += kTailWaves) {
        float xp[16], xq[16];
        load_sub<DT, VEC>(rr, has_q, static_cast<int64_t>(i) * kSub + 16 * lane, a.V, xp, xq);
        double tr = 0.0;
        float tpf = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float ep = t_of_p(xp[v], rr, c32);
            tpf += ep;
            tr += resid_t(static_cast<double>(ep), xq[v], has_q, c32, rr);
        }
        tr = wave_sum(tr);
        const double tp = wave_sum(static_cast<double>(tpf));
        if (lane == 0) {
            a.sub_r[b * a.nsub + i] = tr;
            a.sub_p[b * a.nsub + i] = tp;
        }
    }
}

// --------------------------------------------------------------------------
// k_draw: one wavefront per sequence. Wave scans of the subsegment masses
// give Z and the subsegment holding u*Z; a scan over that subsegment's 1024
// elements (16 per lane, in registers) gives the first index whose cumulative
// mass exceeds u*Z. If rounding leaves no residual mass at a rejected row the
// draw is made from p_k instead (its masses come from the same pass).
// --------------------------------------------------------------------------
struct DrawArgs {
    int32_t gamma, V, nsub;
    float c32;
    uint64_t seed;
    int64_t b_offset;
    const SeqInfo* info;
    const double* sub_r;
    const double* sub_p;
    int32_t* out_tokens;
    double* dbg_z;
};

__device__ inline double wave_scan(double v, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double y = __shfl_up(v, o, kWave);
        if (lane >= o) v += y;
    }
    return v;
}

// Total of m[0, n) in the order the search below accumulates it.
__device__ inline double scan_total(const double* m, int32_t n, int lane) {
    double base = 0.0;
    for (int32_t t0 = 0; t0 < n; t0 += kWave) {
        const double v = t0 + lane < n ? m[t0 + lane] : 0.0;
        base += __shfl(wave_scan(v, lane), kWave - 1, kWave);
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
        const double v = t0 + lane < n ? m[t0 + lane] : 0.0;
        const double incl = base + wave_scan(v, lane);
        const double prev = __shfl_up(incl, 1, kWave);
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
        base = __shfl(incl, kWave - 1, kWave);
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
        base = __shfl(incl[t], kWave - 1, kWave);
    }
    return base;
}

__device__ inline int32_t regs_find(const double* v, const double* incl, double t, int lane, double& before) {
    int32_t last = -1;
    double last_before = 0.0;
#pragma unroll
    for (int k = 0; k < kDrawTiles; ++k) {
        const double prev = __shfl_up(incl[k], 1, kWave);
        const double base = k == 0 ? 0.0 : __shfl(incl[k - 1], kWave - 1, kWave);
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

template <int DT, bool VEC>
__global__ __launch_bounds__(kWave) void k_draw(const void* __restrict__ tgt, const void* __restrict__ dft,
                                                DrawArgs d) {
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x;
    const SeqInfo in = d.info[b];
    if (in.k < 0) {
        if (d.dbg_z && lane == 0) d.dbg_z[b] = NAN;
        return;
    }
    const int32_t nsub = d.nsub;
    const double* sr = d.sub_r + b * nsub;
    const double* sp = d.sub_p + b * nsub;
    const double u = philox_uniform(d.seed, static_cast<uint32_t>(b + d.b_offset), static_cast<uint32_t>(in.k), 1u);
    double Z, target, before = 0.0;
    int32_t sel;
    bool from_p = false;  // no residual mass left by rounding: draw from p_k
    if (nsub <= kDrawTiles * kWave) {
        double v[kDrawTiles], incl[kDrawTiles];
#pragma unroll
        for (int t = 0; t < kDrawTiles; ++t) v[t] = t * kWave + lane < nsub ? sr[t * kWave + lane] : 0.0;
        Z = regs_scan(v, incl, lane);
        from_p = !(Z > 0.0);
        if (from_p) {
#pragma unroll
            for (int t = 0; t < kDrawTiles; ++t) v[t] = t * kWave + lane < nsub ? sp[t * kWave + lane] : 0.0;
            target = u * regs_scan(v, incl, lane);
        } else {
            target = u * Z;
        }
        sel = regs_find(v, incl, target, lane, before);
    } else {
        Z = scan_total(sr, nsub, lane);
        from_p = !(Z > 0.0);
        const double* m = from_p ? sp : sr;
        target = u * (from_p ? scan_total(sp, nsub, lane) : Z);
        sel = scan_find(m, nsub, target, lane, before);
    }
    if (d.dbg_z && lane == 0) d.dbg_z[b] = Z * in.scale_p;
    int32_t* out = d.out_tokens + b * (d.gamma + 1) + in.k;
    if (sel < 0) {  // no mass at all (cannot happen for a usable row); keep the output defined
        if (lane == 0) *out = -1;
        return;
    }
    const ResidRow rr = resid_row<DT>(tgt, dft, in, b, d.gamma, d.V);
    const bool has_q = rr.qrow != nullptr && !from_p;
    const int64_t j0 = static_cast<int64_t>(sel) * kSub + 16 * lane;
    float xp[16], xq[16];
    load_sub<DT, VEC>(rr, has_q, j0, d.V, xp, xq);
    double mv[16];
    double local = 0.0;
    int32_t mylast = -1;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        mv[v] = resid_t(static_cast<double>(t_of_p(xp[v], rr, d.c32)), xq[v], has_q, d.c32, rr);
        local += mv[v];
        if (mv[v] > 0.0) mylast = static_cast<int32_t>(j0 + v);
    }
    const double incl = before + wave_scan(local, lane);
    const double prev = __shfl_up(incl, 1, kWave);
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
            *out = pick >= 0 ? pick : mylast;
        }
    } else {  // rounding: the last element with mass in the subsegment
        const uint64_t mass = __ballot(mylast >= 0);
        const int l = mass ? 63 - __clzll(static_cast<unsigned long long>(mass)) : 0;
        const int32_t pick = __shfl(mylast, l, kWave);
        if (lane == 0) *out = pick;
    }
}

// --------------------------------------------------------------------------
// Row statistics output for spec_row_stats: one wavefront per row.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_merge_rows(Geom g, StatsArgs sa, float* __restrict__ row_max,
                                                       double* __restrict__ row_sumexp) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave;
    if (r >= g.rows) return;
    const RowStat o = fold_row_wave<false>(g, sa, r, threadIdx.x & (kWave - 1));
    if ((threadIdx.x & (kWave - 1)) == 0) {
        row_max[r] = o.m;
        row_sumexp[r] = usable(o.m, o.s) ? o.s : NAN;
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

struct Workspace {
    void* ptr = nullptr;
    size_t bytes = 0;
};

std::mutex g_mu;
std::map<std::pair<int, void*>, Workspace> g_ws;  // (device, stream) -> buffer
std::map<int, int> g_cus;                         // device -> compute units

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Layout {
    Geom g;
    int32_t nsub, nblk, spb;
    size_t off_pm, off_pr, off_ps, off_pi, off_gath, off_info, off_subr, off_subp, bytes;
};

int elem_bytes(int32_t dtype) { return dtype == SPEC_F32 ? 4 : 2; }

// Chunk geometry: vector chunks are 1 KiB; scalar chunks are 64 x 4 elements.
int32_t chunk_elems(int32_t dtype, bool vec) { return vec ? kWave * (16 / elem_bytes(dtype)) : kWave * 4; }

// Wave ranges of about kChunksPerWave chunks (many more waves than the chip
// holds at once, which keeps its tail short), but at least 16 wavefronts per
// compute unit so that small problems still spread over the chip.
Layout plan(int64_t rows_t, int64_t rows, int32_t V, int32_t dtype, bool vec, int32_t B, int cus) {
    Layout L{};
    Geom& g = L.g;
    g.rows_t = rows_t;
    g.rows = rows;
    g.V = V;
    const int32_t CH = chunk_elems(dtype, vec);
    g.nchunk = (V + CH - 1) / CH;
    const int64_t total = rows * g.nchunk;
    const int64_t min_waves = static_cast<int64_t>(cus) * 16;
    int64_t cpw = kChunksPerWave;
    if ((total + cpw - 1) / cpw < min_waves) cpw = (total + min_waves - 1) / min_waves;
    if (cpw < 1) cpw = 1;
    g.cpw = cpw;
    g.nwaves = (total + cpw - 1) / cpw;
    g.maxp = static_cast<int32_t>((g.nchunk + cpw - 1) / cpw + 1);
    // residual pass: one wavefront per subsegment, about as many blocks as the
    // chip holds at once (32 wavefronts per compute unit), split evenly per
    // sequence
    constexpr int tail_waves = kTailBlock / kWave;
    L.nsub = static_cast<int32_t>((static_cast<int64_t>(V) + kSub - 1) / kSub);
    const int64_t nb = B > 0 ? B : 1;
    int64_t nblk = (static_cast<int64_t>(cus) * (32 / tail_waves)) / nb;
    const int64_t max_blk = (L.nsub + tail_waves - 1) / tail_waves;
    if (nblk > max_blk) nblk = max_blk;
    if (nblk < 1) nblk = 1;
    L.spb = static_cast<int32_t>((L.nsub + nblk - 1) / nblk);
    L.nblk = (L.nsub + L.spb - 1) / L.spb;
    const size_t slots = static_cast<size_t>(rows) * g.maxp;
    const size_t subs = static_cast<size_t>(nb) * L.nsub;
    size_t o = 0;
    L.off_pm = o; o = align_up(o + slots * sizeof(float), 256);
    L.off_pr = o; o = align_up(o + slots * sizeof(float), 256);
    L.off_ps = o; o = align_up(o + slots * sizeof(double), 256);
    L.off_pi = o; o = align_up(o + slots * sizeof(int32_t), 256);
    L.off_gath = o; o = align_up(o + static_cast<size_t>(rows) * sizeof(float), 256);
    L.off_info = o; o = align_up(o + static_cast<size_t>(nb) * sizeof(SeqInfo), 256);
    L.off_subr = o; o = align_up(o + subs * sizeof(double), 256);
    L.off_subp = o; o = align_up(o + subs * sizeof(double), 256);
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

// Caller holds g_mu.
int get_workspace(int dev, hipStream_t stream, size_t bytes, char** out) {
    Workspace& ws = g_ws[std::make_pair(dev, static_cast<void*>(stream))];
    if (ws.bytes < bytes) {
        if (ws.ptr) {
            if (hipStreamSynchronize(stream) != hipSuccess) return fail(SPEC_EHIP, "hipStreamSynchronize failed");
            (void)hipFree(ws.ptr);
            ws = Workspace{};
        }
        const size_t want = align_up(bytes + bytes / 4, 1 << 20);
        if (hipMalloc(&ws.ptr, want) != hipSuccess) {
            ws = Workspace{};
            (void)hipGetLastError();
            return fail(SPEC_ENOMEM, "hipMalloc of the workspace failed");
        }
        ws.bytes = want;
    }
    *out = static_cast<char*>(ws.ptr);
    return SPEC_OK;
}

StatsArgs stats_args(const Layout& L, char* ws, float c32) {
    StatsArgs sa{};
    sa.c32 = c32;
    sa.part_m = reinterpret_cast<float*>(ws + L.off_pm);
    sa.part_r = reinterpret_cast<float*>(ws + L.off_pr);
    sa.part_s = reinterpret_cast<double*>(ws + L.off_ps);
    sa.part_i = reinterpret_cast<int32_t*>(ws + L.off_pi);
    sa.gath = reinterpret_cast<float*>(ws + L.off_gath);
    return sa;
}

// Timing events, when asked for, are bound to the kernel dispatches themselves
// (their start and end timestamps), so they add no packets to the stream.
struct Events {
    hipEvent_t stats_start = nullptr, stats_stop = nullptr, last_stop = nullptr;
};

template <int DT, bool VEC>
void launch_stats_t(bool greedy, const void* tgt, const void* dft, const Geom& g, const StatsArgs& sa,
                    hipStream_t st, const Events& ev) {
    const dim3 blocks(static_cast<unsigned>((g.nwaves + kWavesPerBlock - 1) / kWavesPerBlock));
    if (greedy)
        hipExtLaunchKernelGGL((k_stats<DT, VEC, true, false>), blocks, dim3(kBlock), 0, st, ev.stats_start,
                              ev.stats_stop, 0, tgt, dft, g, sa);
    else if (g.tokens)
        hipExtLaunchKernelGGL((k_stats<DT, VEC, false, true>), blocks, dim3(kBlock), 0, st, ev.stats_start,
                              ev.stats_stop, 0, tgt, dft, g, sa);
    else
        hipExtLaunchKernelGGL((k_stats<DT, VEC, false, false>), blocks, dim3(kBlock), 0, st, ev.stats_start,
                              ev.stats_stop, 0, tgt, dft, g, sa);
}

void launch_stats(int32_t dtype, bool vec, bool greedy, const void* tgt, const void* dft, const Geom& g,
                  const StatsArgs& sa, hipStream_t st, const Events& ev = Events{}) {
    if (dtype == SPEC_F32) {
        if (vec) launch_stats_t<SPEC_F32, true>(greedy, tgt, dft, g, sa, st, ev);
        else launch_stats_t<SPEC_F32, false>(greedy, tgt, dft, g, sa, st, ev);
    } else {
        if (vec) launch_stats_t<SPEC_BF16, true>(greedy, tgt, dft, g, sa, st, ev);
        else launch_stats_t<SPEC_BF16, false>(greedy, tgt, dft, g, sa, st, ev);
    }
}

template <int DT, bool VEC>
void launch_tail_t(const void* tgt, const void* dft, const Geom& g, const StatsArgs& sa, const AcceptArgs& a,
                   const DrawArgs& d, hipStream_t st, hipEvent_t stop) {
    const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(a.B) * a.nblk);
    hipExtLaunchKernelGGL((k_accept_resid<DT, VEC>), dim3(blocks), dim3(kTailBlock), a.stage * 20u, st, nullptr,
                          nullptr, 0, tgt, dft, g, sa, a);
    hipExtLaunchKernelGGL((k_draw<DT, VEC>), dim3(static_cast<unsigned>(a.B)), dim3(kWave), 0, st, nullptr, stop, 0,
                          tgt, dft, d);
}

// T > 0: accept + residual masses, then the draw.
void launch_tail(int32_t dtype, bool vec, const void* tgt, const void* dft, const Geom& g, const StatsArgs& sa,
                 const AcceptArgs& a, const DrawArgs& d, hipStream_t st, hipEvent_t stop) {
    if (dtype == SPEC_F32) {
        if (vec) launch_tail_t<SPEC_F32, true>(tgt, dft, g, sa, a, d, st, stop);
        else launch_tail_t<SPEC_F32, false>(tgt, dft, g, sa, a, d, st, stop);
    } else {
        if (vec) launch_tail_t<SPEC_BF16, true>(tgt, dft, g, sa, a, d, st, stop);
        else launch_tail_t<SPEC_BF16, false>(tgt, dft, g, sa, a, d, st, stop);
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

float fold_temperature(float T) { return static_cast<float>(1.4426950408889634 / static_cast<double>(T)); }

int check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SPEC_EHIP, std::string(what) + ": " + hipGetErrorString(e));
    return SPEC_OK;
}

constexpr int64_t kMaxChunks = int64_t(1) << 31;

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
    const bool greedy = temperature == 0.0f;
    const bool vec = (static_cast<int64_t>(V) * elem_bytes(dtype)) % 16 == 0;
    const int64_t rows_t = static_cast<int64_t>(B) * (gamma + 1);
    const int64_t rows = greedy ? rows_t : rows_t + static_cast<int64_t>(B) * gamma;
    std::lock_guard<std::mutex> lk(g_mu);
    return plan(rows_t, rows, V, dtype, vec, B, compute_units(dev)).bytes;
}

void spec_verify_release_workspace(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto& kv : g_ws) {
        if (!kv.second.ptr) continue;
        (void)hipSetDevice(kv.first.first);
        (void)hipStreamSynchronize(static_cast<hipStream_t>(kv.first.second));
        (void)hipFree(kv.second.ptr);
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
    const int64_t es = elem_bytes(dtype);
    const int64_t rows_t = static_cast<int64_t>(B) * (gamma + 1);
    const int64_t rows = greedy ? rows_t : rows_t + static_cast<int64_t>(B) * gamma;
    if (rows * ((V + 255) / 256) >= kMaxChunks) return fail(SPEC_EINVAL, "problem too large");
    const bool vec = (static_cast<int64_t>(V) * es) % 16 == 0 && aligned16(target_logits) &&
                     (greedy || aligned16(draft_logits));
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPEC_EHIP, "hipGetDevice failed");

    std::lock_guard<std::mutex> lk(g_mu);
    Layout L = plan(rows_t, rows, V, dtype, vec, B, compute_units(dev));
    L.g.gamma = gamma;
    L.g.tokens = draft_tokens;
    char* ws = nullptr;
    if (int rc = get_workspace(dev, st, L.bytes, &ws)) return rc;
    const StatsArgs sa = stats_args(L, ws, c32);
    SeqInfo* info = reinterpret_cast<SeqInfo*>(ws + L.off_info);

    AcceptArgs a{};
    a.tokens = draft_tokens;
    a.gath = sa.gath;
    a.B = B; a.gamma = gamma; a.V = V;
    a.nsub = L.nsub; a.nblk = L.nblk; a.spb = L.spb;
    const int seq_slots = (greedy ? gamma + 1 : 2 * gamma + 1) * L.g.maxp;
    a.stage = seq_slots <= kMaxStage ? seq_slots : 0;
    const uint32_t lds = static_cast<uint32_t>(a.stage) * 20u;
    a.c32 = c32;
    a.seed = seed;
    a.b_offset = extras ? extras->b_offset : 0;
    a.out_tokens = out_tokens;
    a.out_n = out_n_accepted;
    a.info = info;
    a.sub_r = reinterpret_cast<double*>(ws + L.off_subr);
    a.sub_p = reinterpret_cast<double*>(ws + L.off_subp);
    if (extras) {
        a.dbg_row_max = extras->row_max;
        a.dbg_row_sumexp = extras->row_sumexp;
        a.dbg_p = extras->p_draft;
        a.dbg_q = extras->q_draft;
        a.dbg_argmax = extras->argmax;
    }
    Events ev;
    if (extras) {
        ev.stats_start = static_cast<hipEvent_t>(extras->events[0]);
        ev.stats_stop = static_cast<hipEvent_t>(extras->events[1]);
        ev.last_stop = static_cast<hipEvent_t>(extras->events[2]);
    }

    launch_stats(dtype, vec, greedy, target_logits, draft_logits, L.g, sa, st, ev);
    if (int rc = check_launch("statistics kernel")) return rc;
    if (greedy) {
        hipExtLaunchKernelGGL(k_accept_greedy, dim3(static_cast<unsigned>(B)), dim3(kBlock), lds, st, nullptr,
                              ev.last_stop, 0, L.g, sa, a);
        if (int rc = check_launch("accept kernel")) return rc;
    } else {
        DrawArgs d{};
        d.gamma = gamma;
        d.V = V;
        d.nsub = L.nsub;
        d.c32 = c32;
        d.seed = seed;
        d.b_offset = a.b_offset;
        d.info = info;
        d.sub_r = a.sub_r;
        d.sub_p = a.sub_p;
        d.out_tokens = out_tokens;
        d.dbg_z = extras ? extras->Z : nullptr;
        launch_tail(dtype, vec, target_logits, draft_logits, L.g, sa, a, d, st, ev.last_stop);
        if (int rc = check_launch("accept/residual and draw kernels")) return rc;
    }
    return SPEC_OK;
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
    if (!(temperature > 0.0f)) return fail(SPEC_EINVAL, "temperature must be > 0");
    if (!logits || !row_max || !row_sumexp) return fail(SPEC_EINVAL, "null pointer argument");
    const float c32 = fold_temperature(temperature);
    if (!(std::isfinite(c32) && c32 > 0.0f)) return fail(SPEC_EINVAL, "temperature out of range");
    if (rows * ((V + 255) / 256) >= kMaxChunks) return fail(SPEC_EINVAL, "problem too large");
    const bool vec = (static_cast<int64_t>(V) * elem_bytes(dtype)) % 16 == 0 && aligned16(logits);
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPEC_EHIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(g_mu);
    const Layout L = plan(rows, rows, V, dtype, vec, 0, compute_units(dev));
    char* ws = nullptr;
    if (int rc = get_workspace(dev, st, L.bytes, &ws)) return rc;
    const StatsArgs sa = stats_args(L, ws, c32);
    launch_stats(dtype, vec, false, logits, nullptr, L.g, sa, st);
    if (int rc = check_launch("statistics kernel")) return rc;
    const unsigned blocks = static_cast<unsigned>((rows + kWavesPerBlock - 1) / kWavesPerBlock);
    k_merge_rows<<<blocks, kBlock, 0, st>>>(L.g, sa, row_max, row_sumexp);
    return check_launch("merge kernel");
}

}  // extern "C"
