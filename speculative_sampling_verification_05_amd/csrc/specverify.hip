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
//  k_stats   one streaming pass over every target and draft row (all the
//            compulsory bytes). Each wavefront owns a contiguous range of
//            1 KiB chunks of the concatenated rows, keeps per lane an online
//            max and a sum of 2^(x*c - R) (R an integer reference, c =
//            log2(e)/T), software-pipelines its 16-byte loads, and flushes one
//            partial per row piece with wave reductions. At T == 0 it tracks
//            the argmax (first index of the maximum) instead.
//  k_accept  one block per (residual segment, sequence). The block merges the
//            sequence's partials through LDS and its first wavefront decides
//            the accept step: lane i gathers the two logits of draft token i,
//            forms alpha in fp64, draws its Philox uniform, and a ballot finds
//            the first rejection k. Every block of the sequence repeats this
//            (a few kilobytes of loads); block 0 writes the accepted tokens and
//            k. Then each block sums the residual max(0, p - q) of row k (or p
//            of the bonus row) over its segment in fp64.
//  k_draw    one block per sequence: a block scan of the segment sums gives
//            Z and the segment holding u*Z; a second scan over that segment's
//            elements, held in registers, gives the first index whose
//            cumulative mass exceeds u*Z.
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
constexpr int kSeg3 = 4096;                               // elements per residual segment
constexpr int kPerThread = kSeg3 / kBlock;                // segment elements per draw thread
constexpr int kMaxMergeSlots = 2048;                      // partials staged in LDS per row run
constexpr float kRUnset = -1.0e30f;                       // lane reference before the first finite value

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
    // Elements at or beyond V read as -inf (no mass, never a maximum).
    __device__ static inline Raw load_masked(const char* row, int64_t c, int lane, int32_t V) {
        if constexpr (VEC) {
            if (c * CH + lane * EPL < V) return load_full(row, c, lane);  // V % EPL == 0 here
            const uint32_t ninf = DT == SPEC_F32 ? 0xFF800000u : 0xFF80FF80u;
            return make_uint4(ninf, ninf, ninf, ninf);
        } else {
            const int64_t j = c * CH + lane;
            float v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = j + k * kWave < V ? load_one<DT>(row, j + k * kWave) : -INFINITY;
            return make_float4(v[0], v[1], v[2], v[3]);
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

// Block-wide fp64 sum (256 threads); the result is returned to every thread.
__device__ inline double block_sum(double v, double* lds) {
    v = wave_sum(v);
    const int wid = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) lds[wid] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int k = 0; k < kWavesPerBlock; ++k) t += lds[k];
    return t;
}

// Block-wide inclusive scan (256 threads) of fp64 values; also returns the
// exclusive prefix (the previous thread's inclusive value) and the block total.
__device__ inline void block_scan(double v, double* lds, double& incl, double& excl, double& total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    double x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    __syncthreads();
    if (lane == kWave - 1) lds[wid] = x;
    __syncthreads();
    double base = 0.0;
    total = 0.0;
#pragma unroll
    for (int k = 0; k < kWavesPerBlock; ++k) {
        if (k < wid) base += lds[k];
        total += lds[k];
    }
    incl = base + x;
    const double prev = __shfl_up(incl, 1, kWave);
    excl = lane == 0 ? base : prev;
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

// Index into draft_tokens of the token row r scores (-1: the bonus row).
__device__ inline int64_t token_of_row(const Geom& g, int64_t r) {
    if (r >= g.rows_t) return r - g.rows_t;  // draft row b*gamma + i
    const int64_t b = r / (g.gamma + 1), i = r - b * (g.gamma + 1);
    return i < g.gamma ? b * g.gamma + i : -1;
}

template <int DT>
__device__ inline const char* row_ptr(const void* tgt, const void* dft, const Geom& g, int64_t r) {
    return r < g.rows_t ? row_at<DT>(tgt, r * g.V) : row_at<DT>(dft, (r - g.rows_t) * g.V);
}

__device__ inline int64_t first_wave(const Geom& g, int64_t r) { return (r * g.nchunk) / g.cpw; }
__device__ inline int pieces_of(const Geom& g, int64_t r) {
    return static_cast<int>(((r + 1) * g.nchunk - 1) / g.cpw - first_wave(g, r) + 1);
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

template <int DT, bool VEC, bool GREEDY>
__global__ __launch_bounds__(kBlock) void k_stats(const void* __restrict__ tgt, const void* __restrict__ dft,
                                                  Geom g, StatsArgs sa) {
    using C = Chunk<DT, VEC>;
    using Raw = typename C::Raw;
    using Lane = typename std::conditional<GREEDY, ArgLane, SoftLane>::type;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x / kWave);
    if (w >= g.nwaves) return;
    const float c = sa.c32;
    const int64_t total = g.rows * g.nchunk;
    int64_t cc = w * g.cpw;
    const int64_t c_end = cc + g.cpw < total ? cc + g.cpw : total;
    const int64_t nfull = g.V / C::CH;  // chunks of a row that are entirely in bounds
    while (cc < c_end) {
        const int64_t r = cc / g.nchunk;
        const int64_t first = r * g.nchunk;
        const int64_t ce = first + g.nchunk < c_end ? first + g.nchunk : c_end;
        const char* row = row_ptr<DT>(tgt, dft, g, r);
        int64_t cr = cc - first;
        const int64_t cr_end = ce - first;
        const int64_t cr_full = cr_end < nfull ? cr_end : nfull;
        Lane st;
        st.init();
        // the logit at this row's draft token, if this piece holds it (K2 gathers nothing)
        const int64_t tix = g.tokens ? token_of_row(g, r) : -1;
        const int32_t tok = tix >= 0 ? g.tokens[tix] : -1;
        const bool holds_tok = tok >= 0 && tok < g.V && tok >= cr * C::CH && tok < cr_end * C::CH;
        const float tok_logit = holds_tok ? load_one<DT>(row, tok) : 0.0f;
        if (cr + kUnroll <= cr_full) {
            // software pipeline with two register buffers used in turn (no copies):
            // one group's loads are in flight while the other is consumed
            Raw qa[kUnroll], qb[kUnroll];
            int64_t ca = cr, cb = 0;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) qa[u] = C::load_full(row, cr + u, lane);
            cr += kUnroll;
            while (true) {
                const bool hb = cr + kUnroll <= cr_full;
                if (hb) {
                    cb = cr;
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u) qb[u] = C::load_full(row, cr + u, lane);
                    cr += kUnroll;
                }
                consume_group<DT, VEC, kUnroll>(st, qa, ca, lane, c);
                if (!hb) break;
                const bool ha = cr + kUnroll <= cr_full;
                if (ha) {
                    ca = cr;
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u) qa[u] = C::load_full(row, cr + u, lane);
                    cr += kUnroll;
                }
                consume_group<DT, VEC, kUnroll>(st, qb, cb, lane, c);
                if (!ha) break;
            }
        }
        for (; cr < cr_end; ++cr) {
            Raw one[1] = {C::load_masked(row, cr, lane, g.V)};
            consume_group<DT, VEC, 1>(st, one, cr, lane, c);
        }
        const int64_t slot = r * g.maxp + (w - first_wave(g, r));
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
                if (holds_tok) sa.gath[r] = tok_logit;
            }
        } else {
            const float M = wave_max(st.m);
            const float Rw = st.R;  // shared by the wave
            const double Sw = wave_sum(st.S);
            if (lane == 0) {
                sa.part_m[slot] = M;
                sa.part_r[slot] = Rw;
                sa.part_s[slot] = Sw;
                if (holds_tok) sa.gath[r] = tok_logit;
            }
        }
        cc = ce;
    }
}

// --------------------------------------------------------------------------
// Merging partials. A row's partials (M_p, R_p, S_p) combine exactly with
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

// Merge rows [r0, r0 + n) into rs[out0 + j]. When their partials fit the
// staging buffer (cap entries) every thread loads one partial, so all loads are
// in flight together; then thread j folds row r0 + j from LDS. Otherwise each
// row is folded straight from memory.
template <bool GREEDY>
__device__ void merge_rows(const Geom& g, const StatsArgs& sa, int64_t r0, int n, int out0, int cap, float* lm,
                           float* lr, double* ls, int32_t* li, RowStat* rs) {
    const int slots = n * g.maxp;
    if (slots <= cap) {
        for (int t = threadIdx.x; t < slots; t += kBlock) {
            const int j = t / g.maxp, k = t % g.maxp;
            const int64_t r = r0 + j;
            const bool live = k < pieces_of(g, r);
            const int64_t at = r * g.maxp + k;
            lm[t] = live ? sa.part_m[at] : -INFINITY;
            if constexpr (GREEDY) {
                li[t] = live ? sa.part_i[at] : INT32_MAX;
            } else {
                lr[t] = live ? sa.part_r[at] : kRUnset;
                ls[t] = live ? sa.part_s[at] : 0.0;
            }
        }
        __syncthreads();
        for (int j = threadIdx.x; j < n; j += kBlock) {
            const int base = j * g.maxp;
            rs[out0 + j] = fold_row<GREEDY>(g.maxp, lm + base, lr + base, ls + base, li + base, sa.c32);
        }
    } else {
        for (int j = threadIdx.x; j < n; j += kBlock) {
            const int64_t at = (r0 + j) * g.maxp;
            rs[out0 + j] = fold_row<GREEDY>(pieces_of(g, r0 + j), sa.part_m + at, sa.part_r + at,
                                            sa.part_s + at, sa.part_i + at, sa.c32);
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
    int32_t B, gamma, V, nseg;
    int32_t stage;  // staged partials per row run (LDS), 0 = none
    float c32;
    uint64_t seed;
    int64_t b_offset;
    int32_t* out_tokens;
    int32_t* out_n;
    SeqInfo* info;
    double* seg;
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

__device__ inline double resid_t(float xp, float xq, bool has_q, float c32, const ResidRow& rr) {
    const double ep = static_cast<double>(__builtin_amdgcn_exp2f(fmaf(xp, c32, -rr.mcp)));
    if (!has_q) return ep;
    const double eq = static_cast<double>(__builtin_amdgcn_exp2f(fmaf(xq, c32, -rr.mcq)));
    return fmax(0.0, fma(-eq, rr.rho, ep));
}

// --------------------------------------------------------------------------
// k_accept. Dynamic LDS holds the staged partials of one row run (doubles
// first, then the float/int arrays) and the merged stats of the sequence.
// --------------------------------------------------------------------------
struct AcceptShared {
    double red[kWavesPerBlock];
    SeqInfo si;
};

template <int DT, bool VEC, bool GREEDY>
__global__ __launch_bounds__(kBlock) void k_accept(const void* __restrict__ tgt, const void* __restrict__ dft,
                                                   Geom g, StatsArgs sa, AcceptArgs a) {
    extern __shared__ __align__(16) char dyn[];
    __shared__ AcceptShared sh;
    const int32_t gamma = a.gamma, V = a.V;
    const int nseg = GREEDY ? 1 : a.nseg;
    const int64_t b = blockIdx.x / nseg;
    const int32_t s = static_cast<int32_t>(blockIdx.x % nseg);
    const int lane = threadIdx.x & (kWave - 1);
    const bool wave0 = threadIdx.x < kWave;
    const int nt = gamma + 1, nd = GREEDY ? 0 : gamma;
    const int stage = a.stage;
    double* ls = reinterpret_cast<double*>(dyn);
    float* lm = reinterpret_cast<float*>(ls + stage);
    float* lr = lm + stage;
    int32_t* li = reinterpret_cast<int32_t*>(lr + stage);
    RowStat* rs = reinterpret_cast<RowStat*>(dyn + ((static_cast<size_t>(stage) * 20 + 15) / 16) * 16);

    // draft token i and its two logits (gathered by the statistics pass), loaded
    // together with the staged partials
    int32_t x = 0;
    float lt = 0.0f, ld = 0.0f;
    if (wave0 && lane < gamma) {
        x = a.tokens[b * gamma + lane];
        if constexpr (!GREEDY) {
            lt = a.gath[b * (gamma + 1) + lane];
            ld = a.gath[g.rows_t + b * gamma + lane];
        }
    }
    const bool tok_ok = x >= 0 && x < V;
    merge_rows<GREEDY>(g, sa, b * (gamma + 1), nt, 0, stage, lm, lr, ls, li, rs);
    if constexpr (!GREEDY) merge_rows<GREEDY>(g, sa, g.rows_t + b * gamma, nd, nt, stage, lm, lr, ls, li, rs);

    if (wave0) {
        const int i = lane;
        const int64_t R = 2 * gamma + 1;
        const bool dbg = s == 0;
        int status = kAcc;
        float mt = NAN, md = NAN;
        double st = NAN, sd = NAN;
        bool ut = false;
        int32_t amax = -1;
        if (i <= gamma) {
            const RowStat t = rs[i];
            mt = t.m;
            if constexpr (GREEDY) {
                amax = t.arg;
                ut = isfinite(mt);
                if (dbg && a.dbg_row_max) a.dbg_row_max[b * R + i] = mt;
                if (dbg && a.dbg_argmax) a.dbg_argmax[b * (gamma + 1) + i] = amax;
            } else {
                st = t.s;
                ut = usable(mt, st);
                if (dbg && a.dbg_row_max) a.dbg_row_max[b * R + i] = mt;
                if (dbg && a.dbg_row_sumexp) a.dbg_row_sumexp[b * R + i] = st;
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
                if (dbg && a.dbg_row_max) a.dbg_row_max[b * R + gamma + 1 + i] = md;
                if (dbg && a.dbg_row_sumexp) a.dbg_row_sumexp[b * R + gamma + 1 + i] = sd;
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
                if (dbg && a.dbg_p) a.dbg_p[b * gamma + i] = p;
                if (dbg && a.dbg_q) a.dbg_q[b * gamma + i] = q;
            }
        }
        const uint64_t stop = __ballot(i < gamma && status != kAcc);
        const int f = stop ? __ffsll(static_cast<unsigned long long>(stop)) - 1 : gamma;
        const int fstat = __shfl(status, f, kWave);
        const bool bonus_ok = __shfl(ut ? 1 : 0, gamma, kWave) != 0;
        const bool invalid = f < gamma ? (fstat == kBad) : !bonus_ok;
        const int k = invalid ? -1 : f;
        if (s == 0) {
            if (i <= gamma) {
                int32_t o = -1;
                if (!invalid) {
                    if (i < k) o = x;
                    else if (GREEDY && i == k) o = amax;
                }
                a.out_tokens[b * (gamma + 1) + i] = o;
            }
            if (i == 0) a.out_n[b] = k;
        }
        if constexpr (!GREEDY) {
            if (!invalid && i == k) {
                const SeqInfo si = seq_info(k, k < gamma, mt, st, md, sd, a.c32);
                sh.si = si;
                if (s == 0) a.info[b] = si;
            } else if (invalid && i == 0) {
                SeqInfo si;
                si.k = -1; si.mcp = 0.0f; si.mcq = 0.0f; si.has_q = 0; si.rho = 0.0; si.scale_p = 0.0;
                sh.si = si;
                if (s == 0) a.info[b] = si;
            }
        }
    }
    if constexpr (!GREEDY) {
        __syncthreads();
        const SeqInfo in = sh.si;
        if (in.k < 0) return;
        // this block's segment of the residual (t units)
        const float c32 = a.c32;
        const ResidRow rr = resid_row<DT>(tgt, dft, in, b, gamma, V);
        const bool has_q = rr.qrow != nullptr;
        const int64_t e0 = static_cast<int64_t>(s) * kSeg3;
        const int64_t e1 = e0 + kSeg3 < V ? e0 + kSeg3 : V;
        double sum = 0.0;
        if constexpr (VEC) {
            // every load of the segment issued before any is consumed
            constexpr int EPL = 16 / ElemBytes<DT>::value;
            constexpr int NI = kSeg3 / (kBlock * EPL);
            uint4 wp[NI], wq[NI];
#pragma unroll
            for (int it = 0; it < NI; ++it) {
                const int64_t e = e0 + (static_cast<int64_t>(it) * kBlock + threadIdx.x) * EPL;
                const bool in_seg = e < e1;
                wp[it] = in_seg ? *reinterpret_cast<const uint4*>(rr.prow + e * ElemBytes<DT>::value) : make_uint4(0, 0, 0, 0);
                wq[it] = in_seg && has_q ? *reinterpret_cast<const uint4*>(rr.qrow + e * ElemBytes<DT>::value)
                                         : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int it = 0; it < NI; ++it) {
                const int64_t e = e0 + (static_cast<int64_t>(it) * kBlock + threadIdx.x) * EPL;
                if (e >= e1) continue;
                float xp[EPL], xq[EPL];
                Chunk<DT, true>::expand(wp[it], xp);
                Chunk<DT, true>::expand(wq[it], xq);
#pragma unroll
                for (int v = 0; v < EPL; ++v) sum += resid_t(xp[v], xq[v], has_q, c32, rr);
            }
        } else {
            for (int64_t e = e0 + threadIdx.x; e < e1; e += kBlock)
                sum += resid_t(load_one<DT>(rr.prow, e), has_q ? load_one<DT>(rr.qrow, e) : 0.0f, has_q, c32, rr);
        }
        const double tot = block_sum(sum, sh.red);
        if (threadIdx.x == 0) a.seg[b * nseg + s] = tot;
    }
}

// --------------------------------------------------------------------------
// k_draw: one block per sequence.
// --------------------------------------------------------------------------
struct DrawArgs {
    int32_t gamma, V, nseg;
    float c32;
    uint64_t seed;
    int64_t b_offset;
    const SeqInfo* info;
    const double* seg;
    int32_t* out_tokens;
    double* dbg_z;
};

struct DrawShared {
    double red[kWavesPerBlock];
    double before;
    int seg, found, last_pos;
};

// Whole block: the first j in [e0, e1) (e1 - e0 <= kSeg3, ascending) whose
// cumulative mass exceeds t; if rounding leaves none, the last j with mass.
// Thread k owns kPerThread consecutive elements, loaded together and kept in
// registers; a block scan locates the owner, which walks its registers.
template <int DT>
__device__ void draw_in_range(const ResidRow& rr, bool has_q, float c32, int64_t e0, int64_t e1, double t,
                              DrawShared& sh, int32_t* out) {
    const int64_t j0 = e0 + static_cast<int64_t>(threadIdx.x) * kPerThread;
    float xp[kPerThread], xq[kPerThread];
#pragma unroll
    for (int v = 0; v < kPerThread; ++v) {
        const bool in = j0 + v < e1;
        xp[v] = in ? load_one<DT>(rr.prow, j0 + v) : -INFINITY;
        xq[v] = in && has_q ? load_one<DT>(rr.qrow, j0 + v) : 0.0f;
    }
    double m[kPerThread];
    double local = 0.0;
    int32_t mylast = -1;
#pragma unroll
    for (int v = 0; v < kPerThread; ++v) {
        m[v] = j0 + v < e1 ? resid_t(xp[v], xq[v], has_q, c32, rr) : 0.0;
        local += m[v];
        if (m[v] > 0.0) mylast = static_cast<int32_t>(j0 + v);
    }
    if (threadIdx.x == 0) { sh.found = 0; sh.last_pos = -1; }
    double incl, excl, tot;
    block_scan(local, sh.red, incl, excl, tot);  // its barriers also publish the resets above
    if (mylast >= 0) atomicMax(&sh.last_pos, mylast);
    if (excl <= t && t < incl) {
        double run = excl;
        int32_t pick = -1;
#pragma unroll
        for (int v = 0; v < kPerThread; ++v) {
            run += m[v];
            if (pick < 0 && m[v] > 0.0 && run > t) pick = static_cast<int32_t>(j0 + v);
        }
        *out = pick >= 0 ? pick : mylast;
        sh.found = 1;
    }
    __syncthreads();
    if (threadIdx.x == 0 && !sh.found) *out = sh.last_pos;
}

// Segment holding `target` among per-segment masses mass(t), t < nseg: sets
// sh.seg and sh.before (the mass of the segments before it). Guard: the last
// segment with mass.
template <typename F>
__device__ void find_segment(int nseg, double target, F mass, DrawShared& sh) {
    if (threadIdx.x == 0) { sh.seg = -1; sh.last_pos = 0; sh.before = 0.0; }
    double base = 0.0;
    for (int t0 = 0; t0 < nseg; t0 += kBlock) {
        const int t = t0 + threadIdx.x;
        const double v = t < nseg ? mass(t) : 0.0;
        double incl, excl, tot;
        block_scan(v, sh.red, incl, excl, tot);
        incl += base;
        excl += base;
        if (t < nseg && v > 0.0) atomicMax(&sh.last_pos, t);
        if (t < nseg && excl <= target && target < incl) { sh.seg = t; sh.before = excl; }
        base += tot;
        __syncthreads();
        if (sh.seg >= 0) break;
    }
    if (sh.seg < 0) {  // rounding: the last segment with mass and the mass before it
        const int chosen = sh.last_pos;
        double bz = 0.0;
        for (int t = threadIdx.x; t < chosen; t += kBlock) bz += mass(t);
        const double before = block_sum(bz, sh.red);
        if (threadIdx.x == 0) { sh.seg = chosen; sh.before = before; }
        __syncthreads();
    }
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_draw(const void* __restrict__ tgt, const void* __restrict__ dft,
                                                 DrawArgs d) {
    __shared__ DrawShared sh;
    const int64_t b = blockIdx.x;
    const int32_t gamma = d.gamma, V = d.V, nseg = d.nseg;
    const double* seg = d.seg + b * nseg;
    // the sequence's record and (for up to 256 segments) its segment sums, loaded together
    const SeqInfo in = d.info[b];
    const double v0 = threadIdx.x < nseg ? seg[threadIdx.x] : 0.0;
    if (in.k < 0) {
        if (d.dbg_z && threadIdx.x == 0) d.dbg_z[b] = NAN;
        return;
    }
    const float c32 = d.c32;
    const ResidRow rr = resid_row<DT>(tgt, dft, in, b, gamma, V);
    const bool has_q = rr.qrow != nullptr;
    int32_t* out = d.out_tokens + b * (gamma + 1) + in.k;
    const double u = philox_uniform(d.seed, static_cast<uint32_t>(b + d.b_offset), static_cast<uint32_t>(in.k), 1u);
    double Z;
    if (nseg <= kBlock) {
        double incl, excl;
        block_scan(v0, sh.red, incl, excl, Z);
        if (d.dbg_z && threadIdx.x == 0) d.dbg_z[b] = Z * in.scale_p;
        if (Z > 0.0) {
            const double target = u * Z;
            if (threadIdx.x == 0) { sh.seg = -1; sh.last_pos = 0; }
            __syncthreads();
            if (threadIdx.x < nseg && v0 > 0.0) atomicMax(&sh.last_pos, static_cast<int>(threadIdx.x));
            if (threadIdx.x < nseg && excl <= target && target < incl) { sh.seg = threadIdx.x; sh.before = excl; }
            __syncthreads();
            if (sh.seg < 0) {  // rounding: the last segment with mass and the mass before it
                const int chosen = sh.last_pos;
                const double before = block_sum(threadIdx.x < chosen ? v0 : 0.0, sh.red);
                if (threadIdx.x == 0) { sh.seg = chosen; sh.before = before; }
                __syncthreads();
            }
            const int64_t e0 = static_cast<int64_t>(sh.seg) * kSeg3;
            const int64_t e1 = e0 + kSeg3 < V ? e0 + kSeg3 : V;
            draw_in_range<DT>(rr, has_q, c32, e0, e1, target - sh.before, sh, out);
            return;
        }
    } else {
        double z = 0.0;
        for (int t = threadIdx.x; t < nseg; t += kBlock) z += seg[t];
        Z = block_sum(z, sh.red);
        if (d.dbg_z && threadIdx.x == 0) d.dbg_z[b] = Z * in.scale_p;
        if (Z > 0.0) {
            const double target = u * Z;
            find_segment(nseg, target, [&](int t) -> double { return seg[t]; }, sh);
            const int64_t e0 = static_cast<int64_t>(sh.seg) * kSeg3;
            const int64_t e1 = e0 + kSeg3 < V ? e0 + kSeg3 : V;
            draw_in_range<DT>(rr, has_q, c32, e0, e1, target - sh.before, sh, out);
            return;
        }
    }
    // rounding left no residual mass at a rejected row: draw from p_k, with the
    // segment masses of p formed here (a rare, slow path)
    auto pmass = [&](int t) -> double {
        const int64_t e0 = static_cast<int64_t>(t) * kSeg3;
        const int64_t e1 = e0 + kSeg3 < V ? e0 + kSeg3 : V;
        double acc = 0.0;
        for (int64_t j = e0; j < e1; ++j) acc += resid_t(load_one<DT>(rr.prow, j), 0.0f, false, c32, rr);
        return acc;
    };
    double zp = 0.0;
    for (int t = threadIdx.x; t < nseg; t += kBlock) zp += pmass(t);
    const double target = u * block_sum(zp, sh.red);
    find_segment(nseg, target, pmass, sh);
    const int64_t e0 = static_cast<int64_t>(sh.seg) * kSeg3;
    const int64_t e1 = e0 + kSeg3 < V ? e0 + kSeg3 : V;
    draw_in_range<DT>(rr, false, c32, e0, e1, target - sh.before, sh, out);
}

// --------------------------------------------------------------------------
// Row statistics output for spec_row_stats: one thread per row.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_merge_rows(Geom g, StatsArgs sa, float* __restrict__ row_max,
                                                       double* __restrict__ row_sumexp) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (r >= g.rows) return;
    const int64_t at = r * g.maxp;
    const RowStat o = fold_row<false>(pieces_of(g, r), sa.part_m + at, sa.part_r + at, sa.part_s + at,
                                      sa.part_i + at, sa.c32);
    row_max[r] = o.m;
    row_sumexp[r] = usable(o.m, o.s) ? o.s : NAN;
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
    int32_t nseg3;
    size_t off_pm, off_pr, off_ps, off_pi, off_gath, off_info, off_seg, bytes;
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
    L.nseg3 = (V + kSeg3 - 1) / kSeg3;
    const size_t slots = static_cast<size_t>(rows) * g.maxp;
    const size_t nb = static_cast<size_t>(B > 0 ? B : 1);
    size_t o = 0;
    L.off_pm = o; o = align_up(o + slots * sizeof(float), 256);
    L.off_pr = o; o = align_up(o + slots * sizeof(float), 256);
    L.off_ps = o; o = align_up(o + slots * sizeof(double), 256);
    L.off_pi = o; o = align_up(o + slots * sizeof(int32_t), 256);
    L.off_gath = o; o = align_up(o + static_cast<size_t>(rows) * sizeof(float), 256);
    L.off_info = o; o = align_up(o + nb * sizeof(SeqInfo), 256);
    L.off_seg = o; o = align_up(o + nb * L.nseg3 * sizeof(double), 256);
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
        hipExtLaunchKernelGGL((k_stats<DT, VEC, true>), blocks, dim3(kBlock), 0, st, ev.stats_start, ev.stats_stop, 0,
                              tgt, dft, g, sa);
    else
        hipExtLaunchKernelGGL((k_stats<DT, VEC, false>), blocks, dim3(kBlock), 0, st, ev.stats_start, ev.stats_stop,
                              0, tgt, dft, g, sa);
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
void launch_accept_t(bool greedy, const void* tgt, const void* dft, const Geom& g, const StatsArgs& sa,
                     const AcceptArgs& a, size_t lds, hipStream_t st, hipEvent_t stop) {
    if (greedy) {
        hipExtLaunchKernelGGL((k_accept<DT, VEC, true>), dim3(static_cast<unsigned>(a.B)), dim3(kBlock),
                              static_cast<uint32_t>(lds), st, nullptr, stop, 0, tgt, dft, g, sa, a);
    } else {
        const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(a.B) * a.nseg);
        hipExtLaunchKernelGGL((k_accept<DT, VEC, false>), dim3(blocks), dim3(kBlock), static_cast<uint32_t>(lds), st,
                              nullptr, nullptr, 0, tgt, dft, g, sa, a);
    }
}

void launch_accept(int32_t dtype, bool vec, bool greedy, const void* tgt, const void* dft, const Geom& g,
                   const StatsArgs& sa, const AcceptArgs& a, size_t lds, hipStream_t st, hipEvent_t stop) {
    if (dtype == SPEC_F32) {
        if (vec) launch_accept_t<SPEC_F32, true>(greedy, tgt, dft, g, sa, a, lds, st, stop);
        else launch_accept_t<SPEC_F32, false>(greedy, tgt, dft, g, sa, a, lds, st, stop);
    } else {
        if (vec) launch_accept_t<SPEC_BF16, true>(greedy, tgt, dft, g, sa, a, lds, st, stop);
        else launch_accept_t<SPEC_BF16, false>(greedy, tgt, dft, g, sa, a, lds, st, stop);
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
    const int64_t nseg3 = (V + kSeg3 - 1) / kSeg3;
    if (rows * ((V + 255) / 256) >= kMaxChunks || static_cast<int64_t>(B) * nseg3 > INT32_MAX)
        return fail(SPEC_EINVAL, "problem too large");
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
    a.B = B; a.gamma = gamma; a.V = V; a.nseg = L.nseg3;
    const int run_slots = (gamma + 1) * L.g.maxp;  // the larger of the two row runs
    a.stage = run_slots <= kMaxMergeSlots ? run_slots : 0;
    a.c32 = c32;
    a.seed = seed;
    a.b_offset = extras ? extras->b_offset : 0;
    a.out_tokens = out_tokens;
    a.out_n = out_n_accepted;
    a.info = info;
    a.seg = reinterpret_cast<double*>(ws + L.off_seg);
    if (extras) {
        a.dbg_row_max = extras->row_max;
        a.dbg_row_sumexp = extras->row_sumexp;
        a.dbg_p = extras->p_draft;
        a.dbg_q = extras->q_draft;
        a.dbg_argmax = extras->argmax;
    }
    const int nrows_seq = greedy ? gamma + 1 : 2 * gamma + 1;
    const size_t lds = align_up(static_cast<size_t>(a.stage) * 20, 16) + static_cast<size_t>(nrows_seq) * sizeof(RowStat);
    Events ev;
    if (extras) {
        ev.stats_start = static_cast<hipEvent_t>(extras->events[0]);
        ev.stats_stop = static_cast<hipEvent_t>(extras->events[1]);
        ev.last_stop = static_cast<hipEvent_t>(extras->events[2]);
    }

    launch_stats(dtype, vec, greedy, target_logits, draft_logits, L.g, sa, st, ev);
    if (int rc = check_launch("statistics kernel")) return rc;
    launch_accept(dtype, vec, greedy, target_logits, draft_logits, L.g, sa, a, lds, st, greedy ? ev.last_stop : nullptr);
    if (int rc = check_launch("accept kernel")) return rc;
    if (!greedy) {
        DrawArgs d{};
        d.gamma = gamma;
        d.V = V;
        d.nseg = L.nseg3;
        d.c32 = c32;
        d.seed = seed;
        d.b_offset = a.b_offset;
        d.info = info;
        d.seg = a.seg;
        d.out_tokens = out_tokens;
        d.dbg_z = extras ? extras->Z : nullptr;
        if (dtype == SPEC_F32)
            hipExtLaunchKernelGGL(k_draw<SPEC_F32>, dim3(static_cast<unsigned>(B)), dim3(kBlock), 0, st, nullptr,
                                  ev.last_stop, 0, target_logits, draft_logits, d);
        else
            hipExtLaunchKernelGGL(k_draw<SPEC_BF16>, dim3(static_cast<unsigned>(B)), dim3(kBlock), 0, st, nullptr,
                                  ev.last_stop, 0, target_logits, draft_logits, d);
        if (int rc = check_launch("draw kernel")) return rc;
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
    const unsigned blocks = static_cast<unsigned>((rows + kBlock - 1) / kBlock);
    k_merge_rows<<<blocks, kBlock, 0, st>>>(L.g, sa, row_max, row_sumexp);
    return check_launch("merge kernel");
}

}  // extern "C"
