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
// The path is four stream-ordered kernels:
//  K1 k_stats      one streaming pass over every target and draft row (all the
//                  compulsory bytes). Each wavefront owns a contiguous range of
//                  1 KiB chunks of the concatenated rows, keeps a per-lane
//                  online max / sum of 2^(x*c - ref) and flushes one (max, sum)
//                  partial per row piece with wave reductions. No LDS, no
//                  barriers, no atomics. At T == 0 it tracks the argmax instead.
//  K2 k_accept     one wavefront per sequence, one lane per drafted position:
//                  merges the partials, gathers the two logits of the draft
//                  token, forms alpha in fp64, draws the Philox uniform and
//                  finds the first rejection with a ballot.
//  K3a k_resid     per (segment, sequence) fp64 sums of r = max(0, p - q) over
//                  the rejected row (or of p over the bonus row).
//  K3b k_draw      per sequence: pick the segment whose running sum crosses
//                  u*Z, recompute r there, block prefix scan (wave shuffles +
//                  LDS), emit the first index whose cumulative mass exceeds u*Z.
// Exponentials are fp32 (v_exp_f32 through exp2 with c = log2(e)/T folded
// into one FMA); every sum that decides a token is fp64.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "specverify.h"

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kUnroll = 4;          // chunks loaded before any is consumed (K1)
constexpr int kMinChunksPerWave = 4;
constexpr int kSeg3 = 4096;         // elements per residual segment (K3)

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

// A chunk is 64 lanes x EPL elements. Vector path (rows 16-byte aligned): lane l
// holds elements [l*EPL, l*EPL+EPL) from one 16-byte load. Scalar path: lane l
// holds elements l, l+64, l+128, l+192. Either way each lane sees its elements
// in ascending index order.
template <int DT, bool VEC> struct Chunk {
    static constexpr int EPL = VEC ? 16 / ElemBytes<DT>::value : 4;
    static constexpr int CH = kWave * EPL;
    float x[EPL];

    __device__ inline void load_full(const char* row, int64_t c, int lane) {
        if constexpr (VEC) {
            const uint4 w = *reinterpret_cast<const uint4*>(row + (c * CH + lane * EPL) * ElemBytes<DT>::value);
            if constexpr (DT == SPEC_F32) {
                x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
                x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
            } else {
                x[0] = __uint_as_float(w.x << 16); x[1] = __uint_as_float(w.x & 0xFFFF0000u);
                x[2] = __uint_as_float(w.y << 16); x[3] = __uint_as_float(w.y & 0xFFFF0000u);
                x[4] = __uint_as_float(w.z << 16); x[5] = __uint_as_float(w.z & 0xFFFF0000u);
                x[6] = __uint_as_float(w.w << 16); x[7] = __uint_as_float(w.w & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int v = 0; v < EPL; ++v) x[v] = load_one<DT>(row, c * CH + lane + kWave * v);
        }
    }
    // Elements at or beyond V read as -inf (no mass, never a maximum).
    __device__ inline void load_masked(const char* row, int64_t c, int lane, int32_t V) {
        if constexpr (VEC) {
            if (c * CH + lane * EPL < V) {  // V is a multiple of EPL on this path
                load_full(row, c, lane);
            } else {
#pragma unroll
                for (int v = 0; v < EPL; ++v) x[v] = -INFINITY;
            }
        } else {
#pragma unroll
            for (int v = 0; v < EPL; ++v) {
                const int64_t j = c * CH + lane + kWave * v;
                x[v] = j < V ? load_one<DT>(row, j) : -INFINITY;
            }
        }
    }
    __device__ inline int64_t index_of(int64_t c, int lane, int v) const {
        return VEC ? c * CH + lane * EPL + v : c * CH + lane + kWave * v;
    }
};

// --------------------------------------------------------------------------
// Wave reductions (64 lanes)
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

// Geometry of the statistics pass: rows [0, rows_t) are target rows in memory
// order, rows [rows_t, rows) draft rows; each row is nchunk chunks; wave w owns
// chunks [w*cpw, (w+1)*cpw) of the concatenation; row r's partials sit at
// r*maxp + (w - first wave of r).
struct StatsGeom {
    int64_t rows_t;
    int64_t rows;
    int32_t V;
    int32_t nchunk;
    int64_t cpw;
    int64_t nwaves;
    int32_t maxp;
};

template <int DT>
__device__ inline const char* row_ptr(const void* tgt, const void* dft, const StatsGeom& g, int64_t r) {
    return r < g.rows_t ? row_at<DT>(tgt, r * g.V) : row_at<DT>(dft, (r - g.rows_t) * g.V);
}

// --------------------------------------------------------------------------
// K1, T > 0: per-lane online softmax statistics. Lane state: m = max seen,
// mc = fl(m*c) (the reference; 0 while m = -inf), S = sum 2^(fl(x*c - mc)) in
// fp64 (fp32 per chunk group). The wave flush rebases every lane to the wave
// max M exactly in fp64: S_lane * 2^(mc - M*c), M*c formed exactly in fp64.
// --------------------------------------------------------------------------
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_stats(const void* __restrict__ tgt,
                                                  const void* __restrict__ dft, StatsGeom g,
                                                  float c32, float* __restrict__ part_m,
                                                  double* __restrict__ part_s) {
    using C = Chunk<DT, VEC>;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x / kWave);
    if (w >= g.nwaves) return;
    const int64_t total = g.rows * g.nchunk;
    int64_t c = w * g.cpw;
    const int64_t c_end = c + g.cpw < total ? c + g.cpw : total;
    const int32_t nfull = g.V / C::CH;  // chunks of a row that are entirely in bounds
    while (c < c_end) {
        const int64_t r = c / g.nchunk;
        const int64_t first = r * g.nchunk;
        const int64_t ce = first + g.nchunk < c_end ? first + g.nchunk : c_end;
        const char* row = row_ptr<DT>(tgt, dft, g, r);
        float m = -INFINITY, mc = 0.0f;
        double S = 0.0;
        int64_t cr = c - first;
        const int64_t cr_end = ce - first;
        const int64_t cr_full = cr_end < nfull ? cr_end : nfull;
        for (; cr + kUnroll <= cr_full; cr += kUnroll) {
            C ch[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) ch[u].load_full(row, cr + u, lane);
            float cm = ch[0].x[0];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int v = 0; v < C::EPL; ++v) cm = fmaxf(cm, ch[u].x[v]);
            if (cm > m) {
                const float nmc = cm * c32;
                if (S != 0.0) S *= exp2(static_cast<double>(mc) - static_cast<double>(nmc));
                m = cm;
                mc = nmc;
            }
            float acc = 0.0f;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int v = 0; v < C::EPL; ++v) acc += __builtin_amdgcn_exp2f(fmaf(ch[u].x[v], c32, -mc));
            S += static_cast<double>(acc);
        }
        for (; cr < cr_end; ++cr) {
            C ch;
            ch.load_masked(row, cr, lane, g.V);
            float cm = ch.x[0];
#pragma unroll
            for (int v = 1; v < C::EPL; ++v) cm = fmaxf(cm, ch.x[v]);
            if (cm > m) {
                const float nmc = cm * c32;
                if (S != 0.0) S *= exp2(static_cast<double>(mc) - static_cast<double>(nmc));
                m = cm;
                mc = nmc;
            }
            float acc = 0.0f;
#pragma unroll
            for (int v = 0; v < C::EPL; ++v) acc += __builtin_amdgcn_exp2f(fmaf(ch.x[v], c32, -mc));
            S += static_cast<double>(acc);
        }
        const float M = wave_max(m);
        const double contrib =
            S == 0.0 ? 0.0
                     : S * exp2(static_cast<double>(mc) - static_cast<double>(M) * static_cast<double>(c32));
        const double Ssum = wave_sum(contrib);
        if (lane == 0) {
            const int64_t slot = r * g.maxp + (w - first / g.cpw);
            part_m[slot] = M;
            part_s[slot] = Ssum;
        }
        c = ce;
    }
}

// --------------------------------------------------------------------------
// K1, T == 0: per-lane argmax (first index of the maximum) and a NaN flag.
// --------------------------------------------------------------------------
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_argmax(const void* __restrict__ tgt, StatsGeom g,
                                                   float* __restrict__ part_m,
                                                   int32_t* __restrict__ part_i) {
    using C = Chunk<DT, VEC>;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x / kWave);
    if (w >= g.nwaves) return;
    const int64_t total = g.rows * g.nchunk;
    int64_t c = w * g.cpw;
    const int64_t c_end = c + g.cpw < total ? c + g.cpw : total;
    const int32_t nfull = g.V / C::CH;
    while (c < c_end) {
        const int64_t r = c / g.nchunk;
        const int64_t first = r * g.nchunk;
        const int64_t ce = first + g.nchunk < c_end ? first + g.nchunk : c_end;
        const char* row = row_at<DT>(tgt, r * g.V);
        float best = -INFINITY;
        int32_t at = INT32_MAX;
        bool nan = false;
        int64_t cr = c - first;
        const int64_t cr_end = ce - first;
        const int64_t cr_full = cr_end < nfull ? cr_end : nfull;
        for (; cr + kUnroll <= cr_full; cr += kUnroll) {
            C ch[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) ch[u].load_full(row, cr + u, lane);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int v = 0; v < C::EPL; ++v) {
                    const float x = ch[u].x[v];
                    nan |= (x != x);
                    if (x > best) { best = x; at = static_cast<int32_t>(ch[u].index_of(cr + u, lane, v)); }
                }
        }
        for (; cr < cr_end; ++cr) {
            C ch;
            ch.load_masked(row, cr, lane, g.V);
#pragma unroll
            for (int v = 0; v < C::EPL; ++v) {
                const float x = ch.x[v];
                nan |= (x != x);
                if (x > best) { best = x; at = static_cast<int32_t>(ch.index_of(cr, lane, v)); }
            }
        }
        // (value desc, index asc) across the wave
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ob = __shfl_xor(best, o, kWave);
            const int32_t oa = __shfl_xor(at, o, kWave);
            if (ob > best || (ob == best && oa < at)) { best = ob; at = oa; }
        }
        const bool any_nan = __ballot(nan) != 0;
        if (lane == 0) {
            const int64_t slot = r * g.maxp + (w - first / g.cpw);
            part_m[slot] = any_nan ? NAN : best;
            part_i[slot] = at;
        }
        c = ce;
    }
}

// --------------------------------------------------------------------------
// Merging a row's partials
// --------------------------------------------------------------------------
__device__ inline void merge_stats(const StatsGeom& g, int64_t r, float c32, const float* part_m,
                                   const double* part_s, float& M, double& S) {
    const int64_t w0 = (r * g.nchunk) / g.cpw;
    const int64_t w1 = ((r + 1) * g.nchunk - 1) / g.cpw;
    const int64_t base = r * g.maxp;
    M = -INFINITY;
    for (int64_t w = w0; w <= w1; ++w) M = fmaxf(M, part_m[base + (w - w0)]);
    S = 0.0;
    const double Mc = static_cast<double>(M) * static_cast<double>(c32);
    for (int64_t w = w0; w <= w1; ++w) {
        const double pm = static_cast<double>(part_m[base + (w - w0)]);
        S += part_s[base + (w - w0)] * exp2(pm * static_cast<double>(c32) - Mc);
    }
}

__device__ inline void merge_argmax(const StatsGeom& g, int64_t r, const float* part_m,
                                    const int32_t* part_i, float& best, int32_t& at, bool& nan) {
    const int64_t w0 = (r * g.nchunk) / g.cpw;
    const int64_t w1 = ((r + 1) * g.nchunk - 1) / g.cpw;
    const int64_t base = r * g.maxp;
    best = -INFINITY;
    at = INT32_MAX;
    nan = false;
    for (int64_t w = w0; w <= w1; ++w) {
        const float v = part_m[base + (w - w0)];
        const int32_t a = part_i[base + (w - w0)];
        nan |= (v != v);
        if (v > best || (v == best && a < at)) { best = v; at = a; }
    }
}

__device__ inline bool usable(float M, double S) {
    return isfinite(M) && isfinite(S) && S > 0.0;
}

// What the residual kernels need about the row they resample.
struct SeqInfo {
    int32_t k;      // emitted position (0..gamma), -1 = invalid sequence
    float mp, mq;   // max logit of the target row k / draft row k
    int32_t pad;
    double sp, sq;  // sum-exp of those rows
};

struct AcceptArgs {
    const int32_t* tokens;
    int32_t B, gamma, V;
    float c32;
    uint64_t seed;
    int64_t b_offset;
    int32_t* out_tokens;
    int32_t* out_n;
    SeqInfo* info;
    float* dbg_row_max;
    double* dbg_row_sumexp;
    double* dbg_p;
    double* dbg_q;
    int32_t* dbg_argmax;
};

// --------------------------------------------------------------------------
// K2: gather, accept, first rejection. One wave per sequence; lane i < gamma
// is drafted position i, lane gamma the bonus row.
// --------------------------------------------------------------------------
template <int DT, bool GREEDY>
__global__ __launch_bounds__(kBlock) void k_accept(const void* __restrict__ tgt,
                                                   const void* __restrict__ dft, StatsGeom g,
                                                   AcceptArgs a, const float* __restrict__ part_m,
                                                   const double* __restrict__ part_s,
                                                   const int32_t* __restrict__ part_i) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t b = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x / kWave);
    if (b >= a.B) return;
    const int32_t gamma = a.gamma;
    const int i = lane;
    const int64_t R = 2 * gamma + 1;
    int status = kAcc;
    float mt = NAN, md = NAN;
    double st = NAN, sd = NAN;
    bool ut = false;
    int32_t amax = -1;
    int32_t x = 0;
    if (i <= gamma) {
        const int64_t rt = b * (gamma + 1) + i;
        if constexpr (GREEDY) {
            bool nan;
            merge_argmax(g, rt, part_m, part_i, mt, amax, nan);
            ut = !nan && isfinite(mt);
            if (a.dbg_row_max) a.dbg_row_max[b * R + i] = mt;
            if (a.dbg_argmax) a.dbg_argmax[b * (gamma + 1) + i] = amax;
        } else {
            merge_stats(g, rt, a.c32, part_m, part_s, mt, st);
            ut = usable(mt, st);
            if (a.dbg_row_max) a.dbg_row_max[b * R + i] = mt;
            if (a.dbg_row_sumexp) a.dbg_row_sumexp[b * R + i] = st;
        }
    }
    if (i < gamma) {
        x = a.tokens[b * gamma + i];
        const bool tok_ok = x >= 0 && x < a.V;
        if constexpr (GREEDY) {
            status = (!ut || !tok_ok) ? kBad : (x == amax ? kAcc : kRej);
        } else {
            const int64_t rd = g.rows_t + b * gamma + i;
            merge_stats(g, rd, a.c32, part_m, part_s, md, sd);
            const bool ud = usable(md, sd);
            if (a.dbg_row_max) a.dbg_row_max[b * R + gamma + 1 + i] = md;
            if (a.dbg_row_sumexp) a.dbg_row_sumexp[b * R + gamma + 1 + i] = sd;
            double p = NAN, q = NAN;
            if (!ut || !ud || !tok_ok) {
                status = kBad;
            } else {
                const double c = static_cast<double>(a.c32);
                const double lt = load_one<DT>(row_at<DT>(tgt, (b * (gamma + 1) + i) * a.V), x);
                const double ld = load_one<DT>(row_at<DT>(dft, (b * gamma + i) * a.V), x);
                p = exp2((lt - static_cast<double>(mt)) * c) / st;
                q = exp2((ld - static_cast<double>(md)) * c) / sd;
                const double alpha = p == 0.0 ? 0.0 : (q == 0.0 ? 1.0 : fmin(1.0, p / q));
                const double u = philox_uniform(a.seed, static_cast<uint32_t>(b + a.b_offset),
                                                static_cast<uint32_t>(i), 0u);
                status = u < alpha ? kAcc : kRej;
            }
            if (a.dbg_p) a.dbg_p[b * gamma + i] = p;
            if (a.dbg_q) a.dbg_q[b * gamma + i] = q;
        }
    }
    const uint64_t stop = __ballot(i < gamma && status != kAcc);
    const int f = stop ? __ffsll(static_cast<unsigned long long>(stop)) - 1 : gamma;
    const int fstat = __shfl(status, f, kWave);
    const bool bonus_ok = __shfl(ut ? 1 : 0, gamma, kWave) != 0;
    const bool invalid = f < gamma ? (fstat == kBad) : !bonus_ok;
    const int k = invalid ? -1 : f;
    if (i <= gamma) {
        int32_t o = -1;
        if (!invalid) {
            if (i < k) o = x;
            else if (GREEDY && i == k) o = amax;
        }
        a.out_tokens[b * (gamma + 1) + i] = o;
    }
    if (i == 0) a.out_n[b] = k;
    if constexpr (!GREEDY) {
        if (!invalid && i == k) {
            SeqInfo s;
            s.k = k; s.mp = mt; s.mq = k < gamma ? md : 0.0f; s.pad = 0;
            s.sp = st; s.sq = k < gamma ? sd : 1.0;
            a.info[b] = s;
        } else if (invalid && i == 0) {
            SeqInfo s;
            s.k = -1; s.mp = 0.0f; s.mq = 0.0f; s.pad = 0; s.sp = 1.0; s.sq = 1.0;
            a.info[b] = s;
        }
    }
}

// Per-row constants of the residual kernels: p_j = 2^(fl(x_j*c - mcp)) * scale_p.
struct ResidRow {
    const char* prow;
    const char* qrow;  // nullptr at the bonus row
    float mcp, mcq;
    double scale_p, scale_q;
};

template <int DT>
__device__ inline ResidRow resid_row(const void* tgt, const void* dft, const SeqInfo& s,
                                     int64_t b, int32_t gamma, int32_t V, float c32) {
    ResidRow rr;
    rr.prow = row_at<DT>(tgt, (b * (gamma + 1) + s.k) * V);
    rr.qrow = s.k < gamma ? row_at<DT>(dft, (b * gamma + s.k) * V) : nullptr;
    const double c = static_cast<double>(c32);
    rr.mcp = s.mp * c32;
    rr.scale_p = exp2(static_cast<double>(rr.mcp) - static_cast<double>(s.mp) * c) / s.sp;
    rr.mcq = s.mq * c32;
    rr.scale_q = exp2(static_cast<double>(rr.mcq) - static_cast<double>(s.mq) * c) / s.sq;
    return rr;
}

__device__ inline void resid_val(float xp, float xq, bool has_q, float c32, const ResidRow& rr,
                                 double& r, double& p) {
    p = static_cast<double>(__builtin_amdgcn_exp2f(fmaf(xp, c32, -rr.mcp))) * rr.scale_p;
    if (has_q) {
        const double q = static_cast<double>(__builtin_amdgcn_exp2f(fmaf(xq, c32, -rr.mcq))) * rr.scale_q;
        r = fmax(0.0, p - q);
    } else {
        r = p;
    }
}

// Block-wide fp64 sum (256 threads); result valid in thread 0.
__device__ inline double block_sum(double v, double* lds) {
    v = wave_sum(v);
    const int wid = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) lds[wid] = v;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0)
        for (int k = 0; k < kWavesPerBlock; ++k) t += lds[k];
    __syncthreads();
    return t;
}

// --------------------------------------------------------------------------
// K3a: per (segment, sequence) sums of r and of p over the resampled row.
// --------------------------------------------------------------------------
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_resid(const void* __restrict__ tgt,
                                                  const void* __restrict__ dft, int32_t gamma,
                                                  int32_t V, int32_t nseg, float c32,
                                                  const SeqInfo* __restrict__ info,
                                                  double* __restrict__ seg_r,
                                                  double* __restrict__ seg_p) {
    __shared__ double lds[kWavesPerBlock];
    const int64_t b = blockIdx.x / nseg;
    const int32_t s = static_cast<int32_t>(blockIdx.x % nseg);
    const SeqInfo in = info[b];
    if (in.k < 0) return;
    const ResidRow rr = resid_row<DT>(tgt, dft, in, b, gamma, V, c32);
    const bool has_q = rr.qrow != nullptr;
    const int64_t e0 = static_cast<int64_t>(s) * kSeg3;
    const int64_t e1 = e0 + kSeg3 < V ? e0 + kSeg3 : V;
    double sr = 0.0, sp = 0.0;
    if constexpr (VEC) {
        constexpr int EPL = 16 / ElemBytes<DT>::value;
        for (int64_t e = e0 + threadIdx.x * EPL; e < e1; e += kBlock * EPL) {
            const uint4 wp = *reinterpret_cast<const uint4*>(rr.prow + e * ElemBytes<DT>::value);
            uint4 wq = wp;
            if (has_q) wq = *reinterpret_cast<const uint4*>(rr.qrow + e * ElemBytes<DT>::value);
            const uint32_t pw[4] = {wp.x, wp.y, wp.z, wp.w};
            const uint32_t qw[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
            for (int v = 0; v < EPL; ++v) {
                float xp, xq;
                if constexpr (DT == SPEC_F32) {
                    xp = __uint_as_float(pw[v]);
                    xq = __uint_as_float(qw[v]);
                } else {
                    xp = __uint_as_float((v & 1) ? (pw[v >> 1] & 0xFFFF0000u) : (pw[v >> 1] << 16));
                    xq = __uint_as_float((v & 1) ? (qw[v >> 1] & 0xFFFF0000u) : (qw[v >> 1] << 16));
                }
                double r, p;
                resid_val(xp, xq, has_q, c32, rr, r, p);
                sr += r;
                sp += p;
            }
        }
    } else {
        for (int64_t e = e0 + threadIdx.x; e < e1; e += kBlock) {
            const float xp = load_one<DT>(rr.prow, e);
            const float xq = has_q ? load_one<DT>(rr.qrow, e) : 0.0f;
            double r, p;
            resid_val(xp, xq, has_q, c32, rr, r, p);
            sr += r;
            sp += p;
        }
    }
    const double tr = block_sum(sr, lds);
    const double tp = block_sum(sp, lds);
    if (threadIdx.x == 0) {
        seg_r[b * nseg + s] = tr;
        seg_p[b * nseg + s] = tp;
    }
}

// --------------------------------------------------------------------------
// K3b: the inverse-CDF draw. One block per sequence.
// --------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kBlock) void k_draw(const void* __restrict__ tgt,
                                                 const void* __restrict__ dft, int32_t gamma,
                                                 int32_t V, int32_t nseg, float c32, uint64_t seed,
                                                 int64_t b_offset, const SeqInfo* __restrict__ info,
                                                 const double* __restrict__ seg_r,
                                                 const double* __restrict__ seg_p,
                                                 int32_t* __restrict__ out_tokens,
                                                 double* __restrict__ dbg_z) {
    __shared__ double wave_tot[kWavesPerBlock];
    __shared__ double sh_t;
    __shared__ int sh_seg, sh_use_p, sh_found, sh_last;
    const int64_t b = blockIdx.x;
    const SeqInfo in = info[b];
    if (in.k < 0) {
        if (dbg_z && threadIdx.x == 0) dbg_z[b] = NAN;
        return;
    }
    if (threadIdx.x == 0) {
        double Z = 0.0;
        for (int s = 0; s < nseg; ++s) Z += seg_r[b * nseg + s];
        if (dbg_z) dbg_z[b] = Z;
        const bool use_p = !(Z > 0.0);  // rounding left no residual mass: draw from p
        const double* seg = use_p ? seg_p + b * nseg : seg_r + b * nseg;
        if (use_p) {
            Z = 0.0;
            for (int s = 0; s < nseg; ++s) Z += seg[s];
        }
        const double u = philox_uniform(seed, static_cast<uint32_t>(b + b_offset),
                                        static_cast<uint32_t>(in.k), 1u);
        const double t = u * Z;
        double run = 0.0;
        int chosen = -1, last_pos = 0;
        double before = 0.0;
        for (int s = 0; s < nseg; ++s) {
            const double nxt = run + seg[s];
            if (seg[s] > 0.0) last_pos = s;
            if (chosen < 0 && nxt > t) { chosen = s; before = run; }
            run = nxt;
        }
        if (chosen < 0) {  // rounding guard: the last segment with mass
            chosen = last_pos;
            before = 0.0;
            for (int s = 0; s < chosen; ++s) before += seg[s];
        }
        sh_seg = chosen;
        sh_t = t - before;
        sh_use_p = use_p ? 1 : 0;
        sh_found = 0;
        sh_last = -1;
    }
    __syncthreads();
    const ResidRow rr = resid_row<DT>(tgt, dft, in, b, gamma, V, c32);
    const bool has_q = rr.qrow != nullptr && !sh_use_p;
    const int64_t e0 = static_cast<int64_t>(sh_seg) * kSeg3;
    const int64_t e1 = e0 + kSeg3 < V ? e0 + kSeg3 : V;
    const int64_t per = (e1 - e0 + kBlock - 1) / kBlock;
    const int64_t j0 = e0 + threadIdx.x * per;
    const int64_t j1 = j0 + per < e1 ? j0 + per : e1;
    // this thread's mass, in ascending index order
    double local = 0.0;
    int32_t mylast = -1;
    for (int64_t j = j0; j < j1; ++j) {
        double r, p;
        resid_val(load_one<DT>(rr.prow, j), has_q ? load_one<DT>(rr.qrow, j) : 0.0f, has_q, c32, rr, r, p);
        const double m = sh_use_p ? p : r;
        local += m;
        if (m > 0.0) mylast = static_cast<int32_t>(j);
    }
    // inclusive scan over the block: within the wave, then across waves
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    double incl = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
    }
    if (lane == kWave - 1) wave_tot[wid] = incl;
    __syncthreads();
    double wave_base = 0.0;
    for (int k = 0; k < wid; ++k) wave_base += wave_tot[k];
    incl += wave_base;
    double excl = __shfl_up(incl, 1, kWave);
    if (lane == 0) excl = wave_base;
    const double t = sh_t;
    if (mylast >= 0) atomicMax(&sh_last, mylast);
    if (excl <= t && t < incl) {
        // the crossing lies in this thread's elements
        double run = excl;
        int32_t pick = -1;
        for (int64_t j = j0; j < j1; ++j) {
            double r, p;
            resid_val(load_one<DT>(rr.prow, j), has_q ? load_one<DT>(rr.qrow, j) : 0.0f, has_q, c32, rr, r, p);
            const double m = sh_use_p ? p : r;
            run += m;
            if (m > 0.0 && run > t) { pick = static_cast<int32_t>(j); break; }
        }
        if (pick < 0) pick = mylast;  // rounding guard inside the thread's range
        out_tokens[b * (gamma + 1) + in.k] = pick;
        sh_found = 1;
    }
    __syncthreads();
    if (threadIdx.x == 0 && !sh_found) out_tokens[b * (gamma + 1) + in.k] = sh_last;
}

// --------------------------------------------------------------------------
// Row statistics output for spec_row_stats: one thread per row.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_merge_rows(StatsGeom g, float c32,
                                                       const float* __restrict__ part_m,
                                                       const double* __restrict__ part_s,
                                                       float* __restrict__ row_max,
                                                       double* __restrict__ row_sumexp) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (r >= g.rows) return;
    float M;
    double S;
    merge_stats(g, r, c32, part_m, part_s, M, S);
    row_max[r] = M;
    row_sumexp[r] = usable(M, S) ? S : NAN;
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
std::map<std::pair<int, const void*>, int> g_occ; // (device, kernel) -> resident blocks per CU

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Layout {
    StatsGeom g;
    int32_t nseg3;
    size_t off_pm, off_ps, off_pi, off_info, off_segr, off_segp, total;
};

int elem_bytes(int32_t dtype) { return dtype == SPEC_F32 ? 4 : 2; }

// Chunk geometry: vector chunks are 1 KiB; scalar chunks are 64 x 4 elements.
int32_t chunk_elems(int32_t dtype, bool vec) { return vec ? kWave * (16 / elem_bytes(dtype)) : kWave * 4; }

Layout plan(int64_t rows_t, int64_t rows, int32_t V, int32_t dtype, bool vec, int64_t B,
            int64_t wave_slots) {
    Layout L{};
    StatsGeom& g = L.g;
    g.rows_t = rows_t;
    g.rows = rows;
    g.V = V;
    const int32_t CH = chunk_elems(dtype, vec);
    g.nchunk = (V + CH - 1) / CH;
    const int64_t total = rows * g.nchunk;
    int64_t cpw = (total + wave_slots - 1) / wave_slots;
    if (cpw < kMinChunksPerWave) cpw = kMinChunksPerWave;
    g.cpw = cpw;
    g.nwaves = (total + cpw - 1) / cpw;
    g.maxp = static_cast<int32_t>((g.nchunk + cpw - 1) / cpw + 1);
    L.nseg3 = (V + kSeg3 - 1) / kSeg3;
    const size_t slots = static_cast<size_t>(rows) * g.maxp;
    size_t o = 0;
    L.off_pm = o; o = align_up(o + slots * sizeof(float), 256);
    L.off_ps = o; o = align_up(o + slots * sizeof(double), 256);
    L.off_pi = o; o = align_up(o + slots * sizeof(int32_t), 256);
    L.off_info = o; o = align_up(o + static_cast<size_t>(B) * sizeof(SeqInfo), 256);
    L.off_segr = o; o = align_up(o + static_cast<size_t>(B) * L.nseg3 * sizeof(double), 256);
    L.off_segp = o; o = align_up(o + static_cast<size_t>(B) * L.nseg3 * sizeof(double), 256);
    L.total = o;
    return L;
}

// Resident blocks per CU for a kernel (queried once per device and kernel).
int resident_blocks(int dev, const void* kernel) {
    auto key = std::make_pair(dev, kernel);
    auto it = g_occ.find(key);
    if (it != g_occ.end()) return it->second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kBlock, 0) != hipSuccess || n < 1) n = 1;
    g_occ[key] = n;
    return n;
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
            ws.ptr = nullptr;
            ws.bytes = 0;
        }
        const size_t want = align_up(bytes + bytes / 4, 1 << 20);
        if (hipMalloc(&ws.ptr, want) != hipSuccess) {
            ws.ptr = nullptr;
            (void)hipGetLastError();
            return fail(SPEC_ENOMEM, "hipMalloc of the workspace failed");
        }
        ws.bytes = want;
    }
    *out = static_cast<char*>(ws.ptr);
    return SPEC_OK;
}

template <typename K>
const void* kptr(K k) { return reinterpret_cast<const void*>(k); }

const void* stats_kernel(int32_t dtype, bool vec, bool greedy) {
    if (greedy) {
        if (dtype == SPEC_F32) return vec ? kptr(k_argmax<SPEC_F32, true>) : kptr(k_argmax<SPEC_F32, false>);
        return vec ? kptr(k_argmax<SPEC_BF16, true>) : kptr(k_argmax<SPEC_BF16, false>);
    }
    if (dtype == SPEC_F32) return vec ? kptr(k_stats<SPEC_F32, true>) : kptr(k_stats<SPEC_F32, false>);
    return vec ? kptr(k_stats<SPEC_BF16, true>) : kptr(k_stats<SPEC_BF16, false>);
}

int64_t wave_slots_for(int dev, int32_t dtype, bool vec, bool greedy) {
    const int cus = compute_units(dev);
    const int occ = resident_blocks(dev, stats_kernel(dtype, vec, greedy));
    return static_cast<int64_t>(cus) * occ * kWavesPerBlock;
}

void launch_stats(int32_t dtype, bool vec, const void* tgt, const void* dft, const StatsGeom& g,
                  float c32, float* pm, double* ps, hipStream_t st) {
    const unsigned blocks = static_cast<unsigned>((g.nwaves + kWavesPerBlock - 1) / kWavesPerBlock);
    if (dtype == SPEC_F32) {
        if (vec) k_stats<SPEC_F32, true><<<blocks, kBlock, 0, st>>>(tgt, dft, g, c32, pm, ps);
        else k_stats<SPEC_F32, false><<<blocks, kBlock, 0, st>>>(tgt, dft, g, c32, pm, ps);
    } else {
        if (vec) k_stats<SPEC_BF16, true><<<blocks, kBlock, 0, st>>>(tgt, dft, g, c32, pm, ps);
        else k_stats<SPEC_BF16, false><<<blocks, kBlock, 0, st>>>(tgt, dft, g, c32, pm, ps);
    }
}

void launch_argmax(int32_t dtype, bool vec, const void* tgt, const StatsGeom& g, float* pm,
                   int32_t* pi, hipStream_t st) {
    const unsigned blocks = static_cast<unsigned>((g.nwaves + kWavesPerBlock - 1) / kWavesPerBlock);
    if (dtype == SPEC_F32) {
        if (vec) k_argmax<SPEC_F32, true><<<blocks, kBlock, 0, st>>>(tgt, g, pm, pi);
        else k_argmax<SPEC_F32, false><<<blocks, kBlock, 0, st>>>(tgt, g, pm, pi);
    } else {
        if (vec) k_argmax<SPEC_BF16, true><<<blocks, kBlock, 0, st>>>(tgt, g, pm, pi);
        else k_argmax<SPEC_BF16, false><<<blocks, kBlock, 0, st>>>(tgt, g, pm, pi);
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

float fold_temperature(float T) { return static_cast<float>(1.4426950408889634 / static_cast<double>(T)); }

int check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SPEC_EHIP, std::string(what) + ": " + hipGetErrorString(e));
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
    const bool greedy = temperature == 0.0f;
    const bool vec = (static_cast<int64_t>(V) * elem_bytes(dtype)) % 16 == 0;
    const int64_t rows_t = static_cast<int64_t>(B) * (gamma + 1);
    const int64_t rows = greedy ? rows_t : rows_t + static_cast<int64_t>(B) * gamma;
    std::lock_guard<std::mutex> lk(g_mu);
    return plan(rows_t, rows, V, dtype, vec, B, wave_slots_for(dev, dtype, vec, greedy)).total;
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
    if (rows > (int64_t(1) << 40) / V) return fail(SPEC_EINVAL, "problem too large");
    if (static_cast<int64_t>(B) * ((V + kSeg3 - 1) / kSeg3) > INT32_MAX)
        return fail(SPEC_EINVAL, "problem too large");
    const bool vec = (static_cast<int64_t>(V) * es) % 16 == 0 && aligned16(target_logits) &&
                     (greedy || aligned16(draft_logits));
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPEC_EHIP, "hipGetDevice failed");

    std::lock_guard<std::mutex> lk(g_mu);
    const Layout L = plan(rows_t, rows, V, dtype, vec, B, wave_slots_for(dev, dtype, vec, greedy));
    char* ws = nullptr;
    if (int rc = get_workspace(dev, st, L.total, &ws)) return rc;
    float* pm = reinterpret_cast<float*>(ws + L.off_pm);
    double* ps = reinterpret_cast<double*>(ws + L.off_ps);
    int32_t* pi = reinterpret_cast<int32_t*>(ws + L.off_pi);
    SeqInfo* info = reinterpret_cast<SeqInfo*>(ws + L.off_info);
    double* segr = reinterpret_cast<double*>(ws + L.off_segr);
    double* segp = reinterpret_cast<double*>(ws + L.off_segp);

    auto ev = [&](int k) {
        if (extras && extras->events[k]) (void)hipEventRecord(static_cast<hipEvent_t>(extras->events[k]), st);
    };

    ev(0);
    if (greedy) launch_argmax(dtype, vec, target_logits, L.g, pm, pi, st);
    else launch_stats(dtype, vec, target_logits, draft_logits, L.g, c32, pm, ps, st);
    if (int rc = check_launch("statistics kernel")) return rc;
    ev(1);

    AcceptArgs a{};
    a.tokens = draft_tokens;
    a.B = B; a.gamma = gamma; a.V = V;
    a.c32 = c32;
    a.seed = seed;
    a.b_offset = extras ? extras->b_offset : 0;
    a.out_tokens = out_tokens;
    a.out_n = out_n_accepted;
    a.info = info;
    if (extras) {
        a.dbg_row_max = extras->row_max;
        a.dbg_row_sumexp = extras->row_sumexp;
        a.dbg_p = extras->p_draft;
        a.dbg_q = extras->q_draft;
        a.dbg_argmax = extras->argmax;
    }
    const unsigned kb = static_cast<unsigned>((B + kWavesPerBlock - 1) / kWavesPerBlock);
    if (dtype == SPEC_F32) {
        if (greedy) k_accept<SPEC_F32, true><<<kb, kBlock, 0, st>>>(target_logits, draft_logits, L.g, a, pm, ps, pi);
        else k_accept<SPEC_F32, false><<<kb, kBlock, 0, st>>>(target_logits, draft_logits, L.g, a, pm, ps, pi);
    } else {
        if (greedy) k_accept<SPEC_BF16, true><<<kb, kBlock, 0, st>>>(target_logits, draft_logits, L.g, a, pm, ps, pi);
        else k_accept<SPEC_BF16, false><<<kb, kBlock, 0, st>>>(target_logits, draft_logits, L.g, a, pm, ps, pi);
    }
    if (int rc = check_launch("accept kernel")) return rc;
    ev(2);
    if (greedy) return SPEC_OK;
    const unsigned g3 = static_cast<unsigned>(static_cast<int64_t>(L.nseg3) * B);
    double* dz = extras ? extras->Z : nullptr;
    const int64_t boff = extras ? extras->b_offset : 0;
    if (dtype == SPEC_F32) {
        if (vec) k_resid<SPEC_F32, true><<<g3, kBlock, 0, st>>>(target_logits, draft_logits, gamma, V, L.nseg3, c32, info, segr, segp);
        else k_resid<SPEC_F32, false><<<g3, kBlock, 0, st>>>(target_logits, draft_logits, gamma, V, L.nseg3, c32, info, segr, segp);
    } else {
        if (vec) k_resid<SPEC_BF16, true><<<g3, kBlock, 0, st>>>(target_logits, draft_logits, gamma, V, L.nseg3, c32, info, segr, segp);
        else k_resid<SPEC_BF16, false><<<g3, kBlock, 0, st>>>(target_logits, draft_logits, gamma, V, L.nseg3, c32, info, segr, segp);
    }
    if (int rc = check_launch("residual kernel")) return rc;
    ev(3);
    if (dtype == SPEC_F32)
        k_draw<SPEC_F32><<<static_cast<unsigned>(B), kBlock, 0, st>>>(target_logits, draft_logits, gamma, V, L.nseg3, c32, seed, boff, info, segr, segp, out_tokens, dz);
    else
        k_draw<SPEC_BF16><<<static_cast<unsigned>(B), kBlock, 0, st>>>(target_logits, draft_logits, gamma, V, L.nseg3, c32, seed, boff, info, segr, segp, out_tokens, dz);
    if (int rc = check_launch("draw kernel")) return rc;
    ev(4);
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
    if (rows > (int64_t(1) << 40) / V) return fail(SPEC_EINVAL, "problem too large");
    const bool vec = (static_cast<int64_t>(V) * elem_bytes(dtype)) % 16 == 0 && aligned16(logits);
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SPEC_EHIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(g_mu);
    const Layout L = plan(rows, rows, V, dtype, vec, 1, wave_slots_for(dev, dtype, vec, false));
    char* ws = nullptr;
    if (int rc = get_workspace(dev, st, L.total, &ws)) return rc;
    float* pm = reinterpret_cast<float*>(ws + L.off_pm);
    double* ps = reinterpret_cast<double*>(ws + L.off_ps);
    launch_stats(dtype, vec, logits, nullptr, L.g, c32, pm, ps, st);
    if (int rc = check_launch("statistics kernel")) return rc;
    const unsigned blocks = static_cast<unsigned>((rows + kBlock - 1) / kBlock);
    k_merge_rows<<<blocks, kBlock, 0, st>>>(L.g, c32, pm, ps, row_max, row_sumexp);
    return check_launch("merge kernel");
}

}  // extern "C"
