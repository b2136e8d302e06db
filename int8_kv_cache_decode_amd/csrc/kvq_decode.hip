// kvq_decode.hip -- stream-K single-query decode attention for gfx950.
//
// The rows of every (sequence, live KV head) are cut into 16-row tiles laid
// end to end, and each wave of a grid that is resident all at once takes an
// equal, contiguous share of that tile stream (kvq_internal.h).  Every K and
// V row is read from HBM exactly once and serves all hpk Q heads of the GQA
// group (cortiq-engine 0.3.4 kv_cache.rs, LayerKvCache::attend_group: each
// stored row read once for all heads of its group).  A wave streams its
// share with 16-byte loads, keeps an online-softmax state per Q head in
// registers (franken_ocr 0.8.0 rswa.rs, fold: rescale the running sum and
// accumulator when the running max grows, never materialising the score
// row), and writes one partial (max, sum, acc[128]) per Q head for each
// segment its share touches.  A second kernel merges the partials of a
// (sequence, Q head) with the same rescaling and divides.
//
// Scores are kept in log2 units (the query is pre-scaled by
// log2(e)/sqrt(128)) so every exponential is one v_exp_f32.
#include <math.h>

#include <atomic>
#include <type_traits>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kQScale = 0.12751743082459868f;   // log2(e) / sqrt(128)
constexpr double kQScale64 = 0.12751743082459868;
constexpr int kWaves = 4;   // waves per workgroup

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Streaming loads: K and V rows are read exactly once per call, so they are
// fetched with the non-temporal hint (measured on MI355X: a plain streaming
// read of 335 MB peaks near 6.0 TB/s, the same read with this hint near
// 6.8 TB/s).
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_stream(const float* p) {
    const v4f_t t = __builtin_nontemporal_load(reinterpret_cast<const v4f_t*>(p));
    return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint4 ld_stream(const int8_t* p) {
    const v4u_t t = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ float ld_stream1(const float* p) { return __builtin_nontemporal_load(p); }

// Cross-lane exchanges on the VALU only (no LDS permute): DPP row
// permutations within 16-lane rows, and gfx950's permlane swaps across rows.
// Lane l takes x of another lane of its row (every source lane is inside the
// row, so bound_ctrl never applies while the whole wave is active).
template <int kCtrl>
__device__ __forceinline__ int dpp_row(int x) { return __builtin_amdgcn_mov_dpp(x, kCtrl, 0xf, 0xf, true); }
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]: lane i <- i ^ 1
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]: lane i <- i ^ 2
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <- 15 - i within each 16 lanes
// Rows 2k + 1 of a exchanged with rows 2k of b (16-lane rows): afterwards
// a + b (or max) at every lane combines lanes l and l ^ 16 of the inputs.
__device__ __forceinline__ void swap16(float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
// Upper 32 lanes of a exchanged with the lower 32 of b.
__device__ __forceinline__ void swap32(float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
// Max over the 16 lanes of a row (lanes sharing lane >> 4): quad swaps, then
// the half-row and row mirrors pair whole quads and half-rows.  The max runs
// on integer keys that order like the floats (a negative float's magnitude
// bits flipped), so each step is one v_max_i32 with its DPP operand and needs
// no NaN canonicalisation; the result is exact.  Every lane must be active.
// In the q8 decode's tile loop this replaced four LDS permutes on the path
// from the scores to the weights (batched q8 decode 388.9 -> 381.5 us, int8
// route 360.5 -> 354.1 us on one MI355X).
__device__ __forceinline__ float max16(float x) {
    const int b = __float_as_int(x);
    int k = b ^ ((b >> 31) & 0x7fffffff);
    k = max(k, dpp_row<kDppXor1>(k));
    k = max(k, dpp_row<kDppXor2>(k));
    k = max(k, dpp_row<kDppHalfMirror>(k));
    k = max(k, dpp_row<kDppMirror>(k));
    return __int_as_float(k ^ ((k >> 31) & 0x7fffffff));
}

// Max (sum) of x over lanes l and l ^ 16, then over l and l ^ 32.
__device__ __forceinline__ float max_rows(float x) {
    float a = x, b = x;
    swap16(a, b);
    a = b = fmaxf(a, b);
    swap32(a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float sum_rows(float x) {
    float a = x, b = x;
    swap16(a, b);
    a = b = a + b;
    swap32(a, b);
    return a + b;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// First share [w T / W, (w + 1) T / W) holding tile t.
__host__ __device__ inline int tile_owner(int t, int T, int W) {
    return (int)(((int64_t)(t + 1) * W - 1) / T);
}

// The part of one share that lies in one (sequence, live head) segment.
// A segment's tiles start at its stream start (the first visible row, or for
// the int8 kinds the 16-row boundary at or below it); rows below the first
// visible one are masked.
struct Piece {
    int j, gl, b, g;
    int row0, row1;  // rows of the segment, [row0, row1)
    int lo;          // first visible row of the segment
    int slot;        // partial slot: share + segment index
    size_t hrow;     // first storage row of the (sequence, live head)
    size_t hidx;     // index of the (sequence, live head): b * n_live + gl
};

// First row of a segment's tile stream and its first visible row: a
// decode's stream start and visible-row start, row 0 for a verify.
__device__ __forceinline__ int seg_first(const DecodeArgs& a, int j) { return a.start[j]; }
__device__ __forceinline__ int seg_first(const VerifyArgs&, int) { return 0; }
__device__ __forceinline__ int seg_lo(const DecodeArgs& a, int j) { return a.first[j]; }
__device__ __forceinline__ int seg_lo(const VerifyArgs&, int) { return 0; }

// Calls f(piece) for each piece of share w, in stream order.
template <class Args, class F>
__device__ __forceinline__ void for_each_piece(const Args& a, int w, F&& f) {
    const int T = a.n_tiles, W = a.n_shares;
    int t = (int)((int64_t)w * T / W);
    const int t1 = (int)((int64_t)(w + 1) * T / W);
    // sequence of tile t: the last j with tile_base[j] <= t (it has tiles)
    int lo = 0, hi = a.n_seq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.tile_base[mid] <= t) lo = mid; else hi = mid - 1;
    }
    int j = lo;
    int gl = (t - a.tile_base[j]) / a.ntile[j];
    while (t < t1) {
        const int nt = a.ntile[j];
        const int sb = a.tile_base[j] + gl * nt;
        const int pe = min(t1, sb + nt);
        Piece p;
        p.j = j;
        p.gl = gl;
        p.b = a.seq0 + j;
        p.g = arg_byte(a.live_head, gl);
        p.row0 = seg_first(a, j) + kTileRows * (t - sb);
        p.row1 = min(seg_first(a, j) + kTileRows * (pe - sb), a.len[j]);
        p.lo = seg_lo(a, j);
        p.slot = w + j * a.n_live + gl;
        p.hidx = (size_t)p.b * a.n_live + gl;
        p.hrow = p.hidx * a.capacity;
        f(p);
        t = pe;
        if (t < t1 && ++gl == a.n_live) {   // next segment with tiles
            gl = 0;
            do ++j; while (a.ntile[j] == 0);
        }
    }
}

// Share of the calling wave (wave-uniform): one share per wave.
__device__ __forceinline__ int share_index() {
    return blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// ---------------------------------------------------------------------------
// f32 cache.  Lane layout: half = lane >> 5 picks the row of a pair, seg =
// lane & 31 the 4 channels [4 seg, 4 seg + 4).  One 16-byte load per lane
// covers two consecutive 512-byte rows; a wave takes 16 rows per step.
// ---------------------------------------------------------------------------
// Sum 8 per-lane partials over the 32 lanes of a half so that lanes with
// (seg >> 2) == i end with the total of partial i (transpose-reduce: 9
// exchanges instead of 40).  In this kernel the LDS permutes measured
// faster than the VALU row permutations of the q8 kernel (57.6 vs 58.8 us
// for the 32k R-SWA step): with them the compiler kept only a few of the
// tile's loads in flight.
__device__ __forceinline__ float reduce8_over32(const float (&v)[8], int seg) {
    const bool b4 = seg & 16, b3 = seg & 8, b2 = seg & 4;
    float x[4], y[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float keep = b4 ? v[i + 4] : v[i];
        const float send = b4 ? v[i] : v[i + 4];
        x[i] = keep + __shfl_xor(send, 16, 64);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float keep = b3 ? x[i + 2] : x[i];
        const float send = b3 ? x[i] : x[i + 2];
        y[i] = keep + __shfl_xor(send, 8, 64);
    }
    float z = (b2 ? y[1] : y[0]) + __shfl_xor(b2 ? y[0] : y[1], 4, 64);
    z += __shfl_xor(z, 2, 64);
    z += __shfl_xor(z, 1, 64);
    return z;
}

// Gemma-2 logit soft-cap in log2 units ([P2] attend_group_upto):
// c2 * tanh(s / c2), c2 = softcap * log2 e, in f64 without a library call.
// tanh|y| = (1 - e) / (1 + e) with e = exp(-2|y|) = 2^z, z = n + r, n =
// rint(z), |r| <= 1/2, and 2^r = exp(r ln 2) from its Taylor polynomial of
// degree 10 (truncation below 3e-13 for |r ln 2| <= 0.35): the capped score
// carries a relative error near 1e-12, far below the f32 output's.
__device__ __forceinline__ double soft_cap(double s, double c2, double inv_c2) {
    const double z = -2.0 * 1.4426950408889634 * (fabs(s) * inv_c2);
    const double n = rint(z);
    const double r = (z - n) * 0.6931471805599453;
    double p = 1.0 / 3628800.0;                        // 1/10!
    p = fma(p, r, 1.0 / 362880.0);
    p = fma(p, r, 1.0 / 40320.0);
    p = fma(p, r, 1.0 / 5040.0);
    p = fma(p, r, 1.0 / 720.0);
    p = fma(p, r, 1.0 / 120.0);
    p = fma(p, r, 1.0 / 24.0);
    p = fma(p, r, 1.0 / 6.0);
    p = fma(p, r, 0.5);
    p = fma(p, r, 1.0);
    p = fma(p, r, 1.0);
    const double e = ldexp(p, (int)fmax(n, -2000.0));  // 0 once |y| is large: tanh = 1
    return copysign(c2 * ((1.0 - e) / (1.0 + e)), s);
}

// The fold of one piece of an f32 segment by one wave: the online-softmax
// state per Q head of the group over rows [row0, row1) -- max m and sum l in
// log2 units (l summed over the wave) and the weighted V sum acc, lane l < 32
// holding channels 4 l .. 4 l + 3.  The wave whose piece holds the R-SWA row
// stores it into the ring first (nobody else reads that row).
template <int HPK, bool kCap>
__device__ __forceinline__ void f32_piece(const DecodeArgs& a, const Piece& it, float (&m)[HPK], float (&lsum)[HPK],
                                          float4 (&acc)[HPK]) {
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5, seg = lane & 31;
    const double inv_c2 = kCap ? 1.0 / a.softcap2 : 0.0;
    const float* K = a.k + it.hrow * kHD;
    const float* V = a.v + it.hrow * kHD;
    const int wrow = a.wrow[it.j];
    const bool has_w = wrow >= it.row0 && wrow < it.row1;
    const float* kn = has_w ? a.k_new + ((size_t)it.b * a.n_kv_heads + it.g) * kHD : K;
    const float* vn = has_w ? a.v_new + ((size_t)it.b * a.n_kv_heads + it.g) * kHD : V;

    // R-SWA ring write: this wave's share holds the row, nobody else reads it.
    if (has_w && lane < 32) {
        *(float4*)(a.k_store + (it.hrow + wrow) * kHD + 4 * lane) = *(const float4*)(kn + 4 * lane);
        *(float4*)(a.v_store + (it.hrow + wrow) * kHD + 4 * lane) = *(const float4*)(vn + 4 * lane);
    }

    float4 qv[HPK];
#pragma unroll
    for (int h = 0; h < HPK; ++h) {
        const float4 t = *(const float4*)(a.q + ((size_t)it.b * a.n_q_heads + it.g * HPK + h) * kHD + 4 * seg);
        qv[h] = make_float4(t.x * kQScale, t.y * kQScale, t.z * kQScale, t.w * kQScale);
    }
    float l[HPK];
#pragma unroll
    for (int h = 0; h < HPK; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
        acc[h] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // kF32Tiles 16-row tiles per step: all their loads leave before the
    // step's arithmetic (rows clamped into the piece; a tile that starts
    // past the piece's end is loaded but not computed)
    constexpr int kF32Tiles = 2;
    for (int r = it.row0; r < it.row1; r += kF32Tiles * kTileRows) {
        float4 kx[8 * kF32Tiles], vx[8 * kF32Tiles];
#pragma unroll
        for (int i = 0; i < 8 * kF32Tiles; ++i) {
            const int row = min(r + 2 * i + half, it.row1 - 1);
            const bool wr = has_w && row == wrow;
            kx[i] = ld_stream((wr ? kn : K + (size_t)row * kHD) + 4 * seg);
            vx[i] = ld_stream((wr ? vn : V + (size_t)row * kHD) + 4 * seg);
        }
#pragma unroll
        for (int tt = 0; tt < kF32Tiles; ++tt) {
            const int rt = r + tt * kTileRows;
            if (tt > 0 && rt >= it.row1) break;
            const int myrow = rt + 2 * (seg >> 2) + half;
#pragma unroll
            for (int h = 0; h < HPK; ++h) {
                float part[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float4 kt = kx[8 * tt + i];
                    float d = qv[h].x * kt.x;
                    d = fmaf(qv[h].y, kt.y, d);
                    d = fmaf(qv[h].z, kt.z, d);
                    d = fmaf(qv[h].w, kt.w, d);
                    part[i] = d;
                }
                float sc = reduce8_over32(part, seg);
                if (kCap) sc = (float)soft_cap((double)sc, a.softcap2, inv_c2);
                if (myrow >= it.row1) sc = -INFINITY;
                const float mnew = fmaxf(m[h], wave_max(sc));
                const float alpha = fast_exp2(m[h] - mnew);
                const float p = fast_exp2(sc - mnew);
                l[h] = l[h] * alpha + ((seg & 3) == 0 ? p : 0.0f);
                float4 ac = make_float4(acc[h].x * alpha, acc[h].y * alpha, acc[h].z * alpha, acc[h].w * alpha);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float pi = __shfl(p, half * 32 + 4 * i, 64);
                    const float4 vt = vx[8 * tt + i];
                    ac.x = fmaf(pi, vt.x, ac.x);
                    ac.y = fmaf(pi, vt.y, ac.y);
                    ac.z = fmaf(pi, vt.z, ac.z);
                    ac.w = fmaf(pi, vt.w, ac.w);
                }
                acc[h] = ac;
                m[h] = mnew;
            }
        }
    }
    // sum the two row halves' accumulators, and the sums over the wave
#pragma unroll
    for (int h = 0; h < HPK; ++h) {
        lsum[h] = wave_sum(l[h]);
        acc[h].x += __shfl_xor(acc[h].x, 32, 64);
        acc[h].y += __shfl_xor(acc[h].y, 32, 64);
        acc[h].z += __shfl_xor(acc[h].z, 32, 64);
        acc[h].w += __shfl_xor(acc[h].w, 32, 64);
    }
}

// One wave per SIMD streams the f32 rows (the launch gives one share per
// SIMD); the occupancy hint lets the scheduler keep more of a step's loads
// in flight.  Measured on the 32k R-SWA step: two tiles per step with the
// hint 57.3 us, one tile without it 57.8 us; two tiles without the hint
// 58.8 us, one tile with it 59.1 us.
template <int HPK, bool kCap>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_decode_f32(const DecodeArgs a) {
    const int w = share_index();
    if (w >= a.n_shares) return;
    const int lane = threadIdx.x & 63;
    for_each_piece(a, w, [&](const Piece& it) {
        float m[HPK], l[HPK];
        float4 acc[HPK];
        f32_piece<HPK, kCap>(a, it, m, l, acc);
        // the piece's partial: (max, sum) and the accumulators
#pragma unroll
        for (int h = 0; h < HPK; ++h) {
            const size_t ix = (size_t)it.slot * HPK + h;
            if (lane < 32) *(float4*)(a.ws_acc + ix * kHD + 4 * lane) = acc[h];
            if (lane == 0) {
                a.ws_ml[ix * 2] = m[h];
                a.ws_ml[ix * 2 + 1] = l[h];
            }
        }
    });
}

// ---------------------------------------------------------------------------
// q8 cache.
//
// Scores are computed exactly, on the matrix cores.  The query side of a
// score, q (.) kcol ([P1] attend: score = s_k * <q (.) col_k, k_q>), is split
// once per piece into four balanced base-128 int8 digits relative to a power
// of two per (Q head, K group):
//   qc = 2^(e-27) * (((d0*128 + d1)*128 + d2)*128 + d3),  |error| <= 2^(e-28).
// For a tile of 16 rows and one 32-channel K group, one
// v_mfma_i32_16x16x64_i8 multiplies A = digits (16 = 4 heads x 4 digits, the
// other group of the 64-channel span zeroed) by B = the int8 codes (64
// channels x 16 rows, 16 contiguous bytes per lane) into exact i32 sums; lane
// (head hq = lane >> 4, row n = lane & 15) receives all four digit sums of its
// (head, row), combines them exactly in f64 and adds ks * 2^(e-27) *
// log2(e)/sqrt(128) of each group.  The score stays f64 until the running max
// is subtracted.
//
// The online softmax runs in that (head, row) layout with a lazily refreshed
// max: it moves only when a tile exceeds it by more than kLazy (log2 units),
// so weights stay <= 2^kLazy and the accumulators are rarely rescaled.  Each
// weight times its row's V scale is split exactly into three bf16 parts and
// goes through a per-wave LDS slot to the value pass, which runs on
// v_mfma_f32_16x16x32_bf16 in the V layout -- lane (ri = lane / kVSeg, seg =
// lane % kVSeg) holds rows ri + kVRows * i of each tile and the kVDim
// channels of seg -- with the V codes (exact in bf16) as the A operand of
// each 8-channel block and the weights' parts as the B operand, one column
// per (part, head).  Every KVQ_Q8_FLUSH tiles the three parts of each f32
// accumulator are summed (DPP) and added into f64 accumulators in LDS, and
// the running sum of weights is f64, so a wave's long share adds no error
// that grows with its length.  The V column field is applied once in the
// combine ([P1] attend: acc (.) vcol at the end).
// ---------------------------------------------------------------------------
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
constexpr float kLazy = 8.0f;
// x plus the x of the lanes 4 and 8 above it in its 16-lane row (DPP row
// shifts; lanes past the row's end contribute 0).
__device__ __forceinline__ float add_shl4_shl8(float x) {
    const float a = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x104, 0xf, 0xf, true));
    const float b = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x108, 0xf, 0xf, true));
    return (x + a) + b;
}
// w = hi + mid + lo exactly (w normal): each part is the top 16 bits (sign,
// exponent, 7 mantissa bits: a bf16) of the remainder, and the remainders
// are exact f32 subtractions; the last one has at most 8 significant bits.
__device__ __forceinline__ void bf16_split3(float w, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    const uint32_t h = __float_as_uint(w) & 0xffff0000u;
    const float r1 = w - __uint_as_float(h);
    const uint32_t m = __float_as_uint(r1) & 0xffff0000u;
    const float r2 = r1 - __uint_as_float(m);
    hi = h >> 16;
    mid = m >> 16;
    lo = __float_as_uint(r2) >> 16;
}
// Two f32 values that are exact in bf16 (small integers), packed as bf16 in one dword.
__device__ __forceinline__ uint32_t bf16_pack(float a, float b) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 x = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf2));
}

// V layout of the q8 kernel: lane (ri = lane / 16, seg = lane % 16) owns
// rows ri + 4 i (i < 4) of a 16-row tile and the 8 channels [8 seg, 8 seg + 8),
// one 8-byte load per row.
constexpr int kVRows = 4;
constexpr int kVSeg = 64 / kVRows;
constexpr int kVDim = kHD / kVSeg;
constexpr int kVLoads = 16 / kVRows;
#ifndef KVQ_Q8_TILES
#define KVQ_Q8_TILES 1
#endif
// Tiles between two flushes of the f32 V accumulators into f64.
#ifndef KVQ_Q8_FLUSH
#define KVQ_Q8_FLUSH 16
#endif

__device__ __forceinline__ void unpack(const uint2 x, float (&f)[8]) {
    const uint32_t w[2] = {x.x, x.y};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        f[4 * k + 0] = (float)(int8_t)(w[k] & 0xffu);
        f[4 * k + 1] = (float)(int8_t)((w[k] >> 8) & 0xffu);
        f[4 * k + 2] = (float)(int8_t)((w[k] >> 16) & 0xffu);
        f[4 * k + 3] = (float)((int32_t)w[k] >> 24);
    }
}
typedef unsigned int v2u_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void ld_v(const int8_t* p, uint2& x) {
    const v2u_t t = __builtin_nontemporal_load(reinterpret_cast<const v2u_t*>(p));
    x = make_uint2(t.x, t.y);
}

__device__ __forceinline__ double shfl_xor_f64(double x, int m) {
    const int2 v = *reinterpret_cast<int2*>(&x);
    int2 r;
    r.x = __shfl_xor(v.x, m, 64);
    r.y = __shfl_xor(v.y, m, 64);
    return *reinterpret_cast<double*>(&r);
}

// One balanced base-128 digit: x = 128 * next + digit, digit in [-64, 63].
__device__ __forceinline__ int take_digit(int& x) {
    const int d = ((x + 64) & 127) - 64;
    x = (x - d) >> 7;
    return d;
}

// rint(x / s) with the quotient correctly rounded, as quantize_row_i8 takes
// it ([P3]), for |x / s| <= 128, from y = x * inv (inv = 1 / s correctly
// rounded): y is then within 2^-15 of the rounded quotient, so both round to
// the same integer unless y lies within 2^-14 of a half-integer; there (and
// for a NaN or infinite y) the quotient itself is formed.
__device__ __forceinline__ float rint_div(float x, float s, float inv) {
    const float y = x * inv;
    const float f = y - floorf(y);
    if (!(fabsf(f - 0.5f) >= 6.103515625e-05f)) return rintf(__fdiv_rn(x, s));
    return rintf(y);
}

// Orders this wave's LDS writes before its following LDS reads.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

#ifndef KVQ_Q8_MIN_WAVES
#define KVQ_Q8_MIN_WAVES 3
#endif
#ifndef KVQ_Q8_PRIO
#define KVQ_Q8_PRIO 1
#endif
// progress (sixteenths of the share) at which a wave's priority drops to 2,
// 1, 0: finer toward the end, where the spread left over decides the tail
// (batched q8, same box: quarters 355.9 us, 8 12 14 352.7 us, 6 10 14 353.8,
// 10 13 15 353.4, 2 6 12 356.4)
#ifndef KVQ_Q8_PRIO_STEPS
#define KVQ_Q8_PRIO_STEPS 8, 12, 14
#endif
__device__ constexpr int kPrioStep[3] = {KVQ_Q8_PRIO_STEPS};
template <int HPK, bool kCap, bool kI8, bool kMf>
__global__ __launch_bounds__(256, (HPK <= 4 ? KVQ_Q8_MIN_WAVES : 2)) void k_decode_q8(const DecodeArgs a) {
    constexpr int NB = (HPK + 3) / 4;                 // blocks of 4 heads (MFMA rows = 4 heads x 4 digits)
    // The value pass runs on the matrix cores (kMf) for groups of 4 or 8
    // heads, on the VALU for 1 or 2 (there the MFMA's 16 columns would hold 3
    // or 6 and the register cost lowers occupancy: the R-SWA step on the int8
    // mirror, group 1, 22.4 us on the VALU against 25.6 us).  The launcher
    // takes the VALU instance for short launches too.
    constexpr bool kPvMfma = kMf && HPK >= 4;
    // per wave, two tiles: the bf16 parts of weight * vs, [head][part][row % 4][row / 4]
    __shared__ __attribute__((aligned(8))) uint16_t sm_wb[kPvMfma ? kWaves : 1][2][kPvMfma ? 4 * NB : 1][3][4][4];
    // per wave, two tiles: weight * vs per [row][head] (VALU value pass)
    __shared__ float sm_pw[kPvMfma ? 1 : kWaves][2][16][kPvMfma ? 1 : HPK];
    __shared__ float sm_alpha[kWaves][2][HPK];        // per wave, two tiles: rescale factor per head
    __shared__ double sm_v64[kWaves][HPK][kHD];       // per wave: flushed V accumulators
    // i8 kind, R-SWA: the ring row's fresh K / V codes and their scales
    __shared__ __attribute__((aligned(16))) int8_t sm_ring[kI8 ? kWaves : 1][2][kHD];
    __shared__ float sm_ring_s[kI8 ? kWaves : 1][2];
    // q8 kind: the query digits as A operands [head block][span][row][channel],
    // and the exponent of each (head, K group)
    __shared__ __attribute__((aligned(16))) int8_t sm_dig[kI8 ? 1 : kWaves][kI8 ? 1 : NB][2][16][64];
    __shared__ int sm_ge[kI8 ? 1 : kWaves][kI8 ? 1 : HPK][4];
    // i8 kind: the query codes of each head of the group
    __shared__ __attribute__((aligned(16))) int8_t sm_qc[kI8 ? kWaves : 1][kI8 ? HPK : 1][kHD];
    const int w = share_index();
    if (w >= a.n_shares) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const double inv_c2 = kCap ? 1.0 / a.softcap2 : 0.0;
    const int hq = lane >> 4, n = lane & 15;          // score layout
    const int ri = lane / kVSeg, seg = lane % kVSeg;  // V layout
    // Wave priority by progress: the SIMD issues the oldest ready wave first,
    // so with equal shares the first workgroups on a compute unit would
    // finish long before the last ones and leave the tail of the launch to
    // one wave per SIMD.  Each wave lowers its priority step by step as it
    // passes fixed fractions of its share (kPrioStep), so a wave that has
    // fallen behind is issued first.
    // (A launch-wide progress counter, one device-scope atomic per wave every
    // 4 tiles, made the batched q8 decode four times slower: every wave hits
    // one address.)
    const int share_tiles = max(1, (int)((int64_t)(w + 1) * a.n_tiles / a.n_shares) -
                                       (int)((int64_t)w * a.n_tiles / a.n_shares));
    int done = 0, lvl = 0;
    if (KVQ_Q8_PRIO) __builtin_amdgcn_s_setprio(3);
    auto progress = [&](int tiles) {
        done += tiles;
        if (KVQ_Q8_PRIO && lvl < 3 && 16 * done >= kPrioStep[lvl] * share_tiles) {
            ++lvl;
            if (lvl == 1) __builtin_amdgcn_s_setprio(2);
            else if (lvl == 2) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
        }
    };
    for_each_piece(a, w, [&](const Piece& it) {
        const int8_t* KQ = a.kq + it.hidx * kq_rows(a.capacity) * kHD;   // tile-major K codes
        const float* KS = a.ks + it.hrow * (kI8 ? 1 : kKScales);
        const int8_t* VQ = a.vq + it.hrow * kHD;
        const float* VS = a.vs + it.hrow;
        const bool frz = !kI8 && arg_byte(a.frozen, it.j) != 0;
        const float* kcol = a.kcol + ((size_t)it.b * a.n_live + it.gl) * kHD;

        // [P3] write_decode_step on the int8 mirror: the wave whose piece holds
        // the R-SWA row quantises the step's K and V rows (quantize_row_i8:
        // scale max|x| / 127, 1 for a zero row; codes rounded half to even),
        // stores codes and scales in the cache and keeps them in its LDS slot:
        // its own loads of that tile may predate the store, so the tile takes
        // the row from the slot.  No other wave reads the row.
        int wl = -1;
        if constexpr (kI8) {
            const int wr = a.wrow[it.j];
            if (wr >= it.row0 && wr < it.row1) {
                wl = wr;
                const size_t src = ((size_t)it.b * a.n_kv_heads + it.g) * kHD + 2 * lane;
                const float2 xk = *(const float2*)(a.k_new + src);
                const float2 xv = *(const float2*)(a.v_new + src);
                const float ak = wave_max(fmaxf(fabsf(xk.x), fabsf(xk.y)));
                const float av = wave_max(fmaxf(fabsf(xv.x), fabsf(xv.y)));
                const float sk = ak > 0.0f ? __fdiv_rn(ak, 127.0f) : 1.0f;
                const float sv = av > 0.0f ? __fdiv_rn(av, 127.0f) : 1.0f;
                char2 ck, cv;
                ck.x = (int8_t)(int)fminf(fmaxf(rintf(__fdiv_rn(xk.x, sk)), -127.0f), 127.0f);
                ck.y = (int8_t)(int)fminf(fmaxf(rintf(__fdiv_rn(xk.y, sk)), -127.0f), 127.0f);
                cv.x = (int8_t)(int)fminf(fmaxf(rintf(__fdiv_rn(xv.x, sv)), -127.0f), 127.0f);
                cv.y = (int8_t)(int)fminf(fmaxf(rintf(__fdiv_rn(xv.y, sv)), -127.0f), 127.0f);
                const size_t row = it.hrow + (size_t)wl;
                *(char2*)(&sm_ring[wave][0][2 * lane]) = ck;
                *(char2*)(&sm_ring[wave][1][2 * lane]) = cv;
                *(char2*)(a.kq_store + it.hidx * kq_rows(a.capacity) * kHD + kq_offset(wl, 2 * lane)) = ck;
                *(char2*)(a.vq_store + row * kHD + 2 * lane) = cv;
                if (lane == 0) {
                    sm_ring_s[wave][0] = sk;
                    sm_ring_s[wave][1] = sv;
                    a.ks_store[row] = sk;
                    a.vs_store[row] = sv;
                }
                wave_lds_sync();
            }
        }

        // The piece's 16-row tiles, kTiles per step; the loads of the next step
        // are issued before this step's arithmetic.
        constexpr int kTiles = KVQ_Q8_TILES;
        constexpr int kStep = 16 * kTiles;
        struct Tile {
            uint4 kb2[2];                                  // B operand: 16 channels of row n per span
            float4 ks4;
            float vsn;
            uint2 vx[kVLoads];                             // rows ri + kVRows * i, channels of seg
        };
        // Offsets within the (sequence, head) block are 32-bit (capacity <=
        // 2^24 rows), so the loads take the block's base from scalar registers.
        auto load_tile = [&](int r0, Tile& t) {
            const uint32_t rk = (uint32_t)min(r0 + n, it.row1 - 1);
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) t.kb2[sp] = ld_stream(KQ + kq_offset((int)rk, 64 * sp + 16 * (lane >> 4)));
            // The 4-byte row scales of a 16-row tile fill half a 128-byte
            // line, and the next tile reads the other half: plain loads keep
            // the line in L2 for it.
            if constexpr (kI8)
                t.ks4.x = KS[rk];
            else
                t.ks4 = ld_stream(KS + rk * kKScales);
            t.vsn = VS[rk];
#pragma unroll
            for (int i = 0; i < kVLoads; ++i) {
                const uint32_t rv = (uint32_t)min(r0 + ri + kVRows * i, it.row1 - 1);
                ld_v(VQ + (rv * kHD + kVDim * seg), t.vx[i]);
            }
        };
        auto load_step = [&](int r, Tile (&t)[kTiles]) {
#pragma unroll
            for (int k = 0; k < kTiles; ++k) load_tile(r + 16 * k, t[k]);
        };
        // The query's loads (and the K column field's) go out first, then the
        // first step's tile loads, then the query set-up below (a piece is
        // never empty): the set-up waits for the query alone.  With the
        // query loaded after the tiles, on a short launch -- where every
        // wave's first tiles fill the memory queues at once -- the set-up
        // waited 3 us for it (one 8192-row sequence, 32 Q / 8 KV heads: 4
        // tiles per wave in 8.7 us; the call went from 15.2 to 14.3 us).
        // (Same box, three alternations: batched q8 350.7 against 353.3 us, the
        // soft-cap + sinks call 355.4 against 358.1 us, int8 unchanged at
        // 325.1 us.)
        float2 qraw[HPK];
        float2 kcv = make_float2(1.f, 1.f);
#pragma unroll
        for (int h = 0; h < HPK; ++h)
            qraw[h] = *(const float2*)(a.q + ((size_t)it.b * a.n_q_heads + it.g * HPK + h) * kHD + 2 * lane);
        if constexpr (!kI8) {
            const float2 kc = *(const float2*)(kcol + 2 * lane);   // loaded either way: no branch
            kcv = frz ? kc : kcv;
        }
        int r0 = it.row0;
        Tile ta[kTiles], tb[kTiles];
        load_step(r0, ta);

        // ---- query digits (MFMA A operand) and per-group scales ----
        // One v_mfma_i32_16x16x64_i8 spans 64 channels = two K groups.  A[m][k]:
        // m = lane & 15 = 4 * head + digit, k = 16 * (lane >> 4) + t of the span,
        // so lanes with lane >> 4 in {0, 1} hold the span's first group and lanes
        // {2, 3} its second; each group gets its own product by zeroing the other
        // half of A.
        const bool first_half = (lane >> 4) < 2;
        v4i qa_lo[NB][2], qa_hi[NB][2];                   // [head block][span]
        double gsc[NB][4];                                // for this lane's score head 4 hb + hq
        if constexpr (!kI8) {
            // Lane l takes channels 2 l and 2 l + 1 of every head of the group:
            // qc = q (.) kcol exactly in f64, the group's largest |qc| over the
            // 16 lanes that hold its 32 channels, and the four digits, written
            // into a per-wave LDS copy of the A operands; each lane then reads
            // its 16 digit bytes.  The group exponents go through LDS too.
            const float2 cv = kcv;
#pragma unroll
            for (int h = 0; h < HPK; ++h) {
                const float2 qv = qraw[h];
                const double q0 = (double)qv.x * (double)cv.x, q1 = (double)qv.y * (double)cv.y;   // exact
                double gmax = fmax(fabs(q0), fabs(q1));
#pragma unroll
                for (int msk = 1; msk < 16; msk <<= 1) gmax = fmax(gmax, shfl_xor_f64(gmax, msk));
                int e = 0;
                (void)frexp(gmax, &e);                             // gmax < 2^e
                const double up = ldexp(1.0, 27 - e);
                int x0 = (int)rint(q0 * up), x1 = (int)rint(q1 * up);   // |x| <= 2^27
                char2 dg[4];
                dg[3] = make_char2((int8_t)take_digit(x0), (int8_t)take_digit(x1));
                dg[2] = make_char2((int8_t)take_digit(x0), (int8_t)take_digit(x1));
                dg[1] = make_char2((int8_t)take_digit(x0), (int8_t)take_digit(x1));
                dg[0] = make_char2((int8_t)x0, (int8_t)x1);
                const int c = 2 * lane;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *(char2*)(&sm_dig[wave][h >> 2][c >> 6][4 * (h & 3) + j][c & 63]) = dg[j];
                if ((lane & 15) == 0) sm_ge[wave][h][lane >> 4] = e;
            }
            wave_lds_sync();
#pragma unroll
            for (int hb = 0; hb < NB; ++hb) {
                const int hm = 4 * hb + ((lane & 15) >> 2), kb = lane >> 4;
#pragma unroll
                for (int sp = 0; sp < 2; ++sp) {
                    v4i pk = {0, 0, 0, 0};
                    if (hm < HPK) pk = *(const v4i*)(&sm_dig[wave][hb][sp][lane & 15][16 * kb]);
                    const v4i zero = {0, 0, 0, 0};
                    qa_lo[hb][sp] = first_half ? pk : zero;
                    qa_hi[hb][sp] = first_half ? zero : pk;
#pragma unroll
                    for (int gs = 0; gs < 2; ++gs) {               // score head 4 hb + hq, group 2 sp + gs
                        const int hs = 4 * hb + hq;
                        const int es = hs < HPK ? sm_ge[wave][hs][2 * sp + gs] : 0;
                        gsc[hb][2 * sp + gs] = ldexp(kQScale64, es - 27);
                    }
                }
            }
        } else {
            // ---- query codes ([P3] quantize_row_i8 on each Q head, in f32) ----
            // Lane l quantises channels 2 l and 2 l + 1 of every head of the
            // group (the head's max over the wave) into a per-wave LDS row;
            // then A rows m = 4 * head take the head's codes over all 64
            // channels of a span (one K scale per row, so no group is zeroed),
            // and the rows of digits 1..3 are zero.  gsc[hb][0] = qscale *
            // log2(e)/sqrt(128) of this lane's score head 4 hb + hq.
            float qsh[HPK];
#pragma unroll
            for (int h = 0; h < HPK; ++h) {
                const float2 x = qraw[h];
                const float amax = wave_max(fmaxf(fabsf(x.x), fabsf(x.y)));
                const float qs = amax > 0.0f ? __fdiv_rn(amax, 127.0f) : 1.0f;
                char2 cq;
                cq.x = (int8_t)(int)fminf(fmaxf(rintf(__fdiv_rn(x.x, qs)), -127.0f), 127.0f);
                cq.y = (int8_t)(int)fminf(fmaxf(rintf(__fdiv_rn(x.y, qs)), -127.0f), 127.0f);
                *(char2*)(&sm_qc[wave][h][2 * lane]) = cq;
                qsh[h] = qs;
            }
            wave_lds_sync();
#pragma unroll
            for (int hb = 0; hb < NB; ++hb) {
                const int hm = 4 * hb + ((lane & 15) >> 2), jm = lane & 3, kb = lane >> 4;
#pragma unroll
                for (int sp = 0; sp < 2; ++sp) {
                    v4i pk = {0, 0, 0, 0};
                    if (jm == 0 && hm < HPK) pk = *(const v4i*)(&sm_qc[wave][hm][64 * sp + 16 * kb]);
                    qa_lo[hb][sp] = pk;
                    qa_hi[hb][sp] = pk;
                }
                float qs = qsh[0];
#pragma unroll
                for (int h = 1; h < HPK; ++h)
                    if (h == 4 * hb + hq) qs = qsh[h];
                gsc[hb][0] = (double)qs * kQScale64;
            }
        }

        float m[NB];
        double l[NB];
#pragma unroll
        for (int hb = 0; hb < NB; ++hb) {
            m[hb] = -INFINITY;
            l[hb] = 0.0;
        }
        // f64 accumulators of this lane: entries kOwn * ri + i of the seg's
        // (head, channel) list e = kVDim * head + channel.
        constexpr int kOwn = HPK * kVDim / kVRows;
        auto cell = [&](int i) -> double& {
            const int e = kOwn * ri + i;
            return sm_v64[wave][e / kVDim][kVDim * seg + e % kVDim];
        };
#pragma unroll
        for (int i = 0; i < kOwn; ++i) cell(i) = 0.0;
        // VALU value pass: per-lane f32 accumulators, head h channels kVDim seg ..
        float acc[kPvMfma ? 1 : HPK][kVDim];
#pragma unroll
        for (int h = 0; h < (kPvMfma ? 1 : HPK); ++h)
#pragma unroll
            for (int c = 0; c < kVDim; ++c) acc[h][c] = 0.0f;
        // Value pass on v_mfma_f32_16x16x32_bf16, one per 8-channel block cb
        // (channels 8 m + cb, m = lane % 16) and block of 4 heads: A = the V
        // codes of the lane's four rows ri + 4 i (exact in bf16; K slots 4..7
        // zero), B = the weights times the rows' V scales in three exact bf16
        // parts, column n = 4 part + head.  Lane l accumulates, for its column
        // (part, head) = (l % 16 / 4, l % 4), channels 8 (4 (l / 16) + i) + cb.
        v4f accv[kPvMfma ? NB : 1][8];
#pragma unroll
        for (int hb = 0; hb < (kPvMfma ? NB : 1); ++hb)
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) accv[hb][cb] = v4f{0.f, 0.f, 0.f, 0.f};
        const int bpart = (lane & 15) >> 2, bhead = lane & 3;
        // The three parts summed onto the part-0 lanes (DPP), added into f64;
        // on the VALU path acc summed over the four row groups (a transposing
        // butterfly leaves lane ri with entries [kOwn ri, kOwn ri + kOwn)),
        // added into f64.  Both clear their accumulators.
        auto flush = [&]() {
            if constexpr (!kPvMfma) {
                constexpr int N = HPK * kVDim;
                float y[N / 2], z[kOwn];
#pragma unroll
                for (int i = 0; i < N / 2; ++i) {
                    // lanes 0..31 keep entry i, lanes 32..63 entry i + N / 2
                    float lo = acc[i / kVDim][i % kVDim], hi = acc[(i + N / 2) / kVDim][(i + N / 2) % kVDim];
                    swap32(lo, hi);
                    y[i] = lo + hi;
                }
#pragma unroll
                for (int i = 0; i < kOwn; ++i) {
                    // rows with lane bit 4 clear keep y[i], the others y[i + kOwn]
                    float lo = y[i], hi = y[i + kOwn];
                    swap16(lo, hi);
                    z[i] = lo + hi;
                }
#pragma unroll
                for (int i = 0; i < kOwn; ++i) cell(i) += (double)z[i];
#pragma unroll
                for (int h = 0; h < HPK; ++h)
#pragma unroll
                    for (int c = 0; c < kVDim; ++c) acc[h][c] = 0.0f;
                return;
            }
#pragma unroll
            for (int hb = 0; hb < NB; ++hb) {
                const int h = 4 * hb + bhead;
#pragma unroll
                for (int cb = 0; cb < 8; ++cb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x = add_shl4_shl8(accv[hb][cb][i]);
                        if (bpart == 0 && h < HPK) sm_v64[wave][h][8 * (4 * ri + i) + cb] += (double)x;
                    }
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) accv[hb][cb] = v4f{0.f, 0.f, 0.f, 0.f};
            }
            wave_lds_sync();
        };
        int since_flush = 0;

        int buf = 0;
        auto compute_tile = [&](int r0, const Tile& tc) {
            Tile t = tc;
            if constexpr (kI8) {
                if (wl >= r0 && wl < r0 + 16) {           // the ring row's tile: that row from the LDS slot
                    const int wn = wl - r0;
                    if (n == wn) {
                        t.kb2[0] = *(const uint4*)(&sm_ring[wave][0][16 * (lane >> 4)]);
                        t.kb2[1] = *(const uint4*)(&sm_ring[wave][0][64 + 16 * (lane >> 4)]);
                        t.ks4.x = sm_ring_s[wave][0];
                        t.vsn = sm_ring_s[wave][1];
                    }
                    if (ri == (wn & (kVRows - 1))) {
                        const uint2 x = *(const uint2*)(&sm_ring[wave][1][kVDim * seg]);
#pragma unroll
                        for (int i = 0; i < kVLoads; ++i)
                            if (i == wn / kVRows) t.vx[i] = x;
                    }
                }
            }
            const bool valid = r0 + n >= it.lo && r0 + n < it.row1;
            // ---- scores (exact), softmax weights in the (head, row) layout ----
            bool rescale = false;
#pragma unroll
            for (int hb = 0; hb < NB; ++hb) {
                const v4i zero = {0, 0, 0, 0};
                double sc = 0.0;
                if constexpr (kI8) {
                    // exact integer dot of the codes over both spans
                    v4i dsum = zero;
#pragma unroll
                    for (int sp = 0; sp < 2; ++sp) {
                        const v4i kbv = {(int)t.kb2[sp].x, (int)t.kb2[sp].y, (int)t.kb2[sp].z, (int)t.kb2[sp].w};
                        dsum = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa_lo[hb][sp], kbv, dsum, 0, 0, 0);
                    }
                    sc = (double)dsum[0] * (gsc[hb][0] * (double)t.ks4.x);
                } else {
                    const float ksg[4] = {t.ks4.x, t.ks4.y, t.ks4.z, t.ks4.w};
#pragma unroll
                    for (int sp = 0; sp < 2; ++sp) {
                        const v4i kbv = {(int)t.kb2[sp].x, (int)t.kb2[sp].y, (int)t.kb2[sp].z, (int)t.kb2[sp].w};
#pragma unroll
                        for (int gs = 0; gs < 2; ++gs) {
                            const int g = 2 * sp + gs;
                            const v4i dsum = __builtin_amdgcn_mfma_i32_16x16x64_i8(gs ? qa_hi[hb][sp] : qa_lo[hb][sp],
                                                                                 kbv, zero, 0, 0, 0);
                            const int t1 = dsum[0] * 128 + dsum[1];
                            const int t2 = dsum[2] * 128 + dsum[3];
                            const double x = fma((double)t1, 16384.0, (double)t2);
                            sc = fma(x, (double)ksg[g] * gsc[hb][g], sc);
                        }
                    }
                }
                const int h = 4 * hb + hq;
                if (kCap) sc = soft_cap(sc, a.softcap2, inv_c2);
                if (!valid || h >= HPK) sc = -INFINITY;
                const float tmax = max16((float)sc);
                float mnew = m[hb], alpha = 1.0f;
                if (tmax > m[hb] + kLazy) {               // uniform over the head's 16 lanes
                    mnew = tmax;
                    alpha = fast_exp2(m[hb] - tmax);
                }
                rescale |= __any(alpha != 1.0f);
                const float p = sc == -INFINITY ? 0.0f : fast_exp2((float)(sc - (double)mnew));
                l[hb] = fma(l[hb], (double)alpha, (double)p);
                m[hb] = mnew;
                if (h < HPK) {
                    if constexpr (kPvMfma) {
                        uint32_t ph, pm, pl;
                        bf16_split3(p * t.vsn, ph, pm, pl);
                        sm_wb[wave][buf][h][0][n & 3][n >> 2] = (uint16_t)ph;
                        sm_wb[wave][buf][h][1][n & 3][n >> 2] = (uint16_t)pm;
                        sm_wb[wave][buf][h][2][n & 3][n >> 2] = (uint16_t)pl;
                    } else {
                        sm_pw[wave][buf][n][h] = p * t.vsn;
                    }
                    if (n == 0) sm_alpha[wave][buf][h] = alpha;
                }
            }
            wave_lds_sync();

            // ---- V accumulation in the (row, channel) layout ----
            if constexpr (!kPvMfma) {
                if (rescale) {
#pragma unroll
                    for (int h = 0; h < HPK; ++h) {
                        const float al = sm_alpha[wave][buf][h];
#pragma unroll
                        for (int c = 0; c < kVDim; ++c) acc[h][c] *= al;
                    }
#pragma unroll
                    for (int i = 0; i < kOwn; ++i) cell(i) *= (double)sm_alpha[wave][buf][(kOwn * ri + i) / kVDim];
                }
                // f32 FMA chains of 4 rows per tile between two f64 flushes
#pragma unroll
                for (int i = 0; i < kVLoads; ++i) {
                    float wv[HPK];
#pragma unroll
                    for (int h = 0; h < HPK; ++h) wv[h] = sm_pw[wave][buf][ri + kVRows * i][h];
                    float vf[kVDim];
                    unpack(t.vx[i], vf);
#pragma unroll
                    for (int h = 0; h < HPK; ++h)
#pragma unroll
                        for (int c = 0; c < kVDim; ++c) acc[h][c] = fmaf(wv[h], vf[c], acc[h][c]);
                }
            } else {
            if (rescale) {
#pragma unroll
                for (int hb = 0; hb < NB; ++hb) {
                    const int h = 4 * hb + bhead;
                    const float al = h < HPK ? sm_alpha[wave][buf][h] : 1.0f;
#pragma unroll
                    for (int cb = 0; cb < 8; ++cb) accv[hb][cb] *= al;
                }
#pragma unroll
                for (int i = 0; i < kOwn; ++i) cell(i) *= (double)sm_alpha[wave][buf][(kOwn * ri + i) / kVDim];
            }
            v8bf bw[NB];
#pragma unroll
            for (int hb = 0; hb < NB; ++hb) {
                v4u bu = {0u, 0u, 0u, 0u};
                if (bpart < 3 && 4 * hb + bhead < HPK) {
                    const uint2 x = *(const uint2*)(&sm_wb[wave][buf][4 * hb + bhead][bpart][ri][0]);
                    bu[0] = x.x;
                    bu[1] = x.y;
                }
                bw[hb] = __builtin_bit_cast(v8bf, bu);
            }
            float vf[kVLoads][kVDim];
#pragma unroll
            for (int i = 0; i < kVLoads; ++i) unpack(t.vx[i], vf[i]);
#pragma unroll
            for (int cb = 0; cb < kVDim; ++cb) {
                const v4u au = {bf16_pack(vf[0][cb], vf[1][cb]), bf16_pack(vf[2][cb], vf[3][cb]), 0u, 0u};
                const v8bf av = __builtin_bit_cast(v8bf, au);
#pragma unroll
                for (int hb = 0; hb < NB; ++hb)
                    accv[hb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bw[hb], accv[hb][cb], 0, 0, 0);
            }
            }
            buf ^= 1;
            if (++since_flush == KVQ_Q8_FLUSH) {
                flush();
                since_flush = 0;
            }
        };

        // Two register sets, ping-pong: the next step's loads are issued before
        // this step's arithmetic.  Rows are clamped into the piece, so a
        // prefetch past its end re-reads its last row (and is unused).  Only
        // steps that start inside the piece are computed, so a step's first
        // tile needs no branch; and the loop leaves only at its head.  Both
        // keep every path through the loop waiting for exactly the loads it
        // consumes: a path that skipped a tile, or a break between the two
        // halves, makes the compiler drain every load at the loop head, so
        // the next step's loads would wait for the current step's.
        auto compute_step = [&](int r, const Tile (&t)[kTiles]) {
#pragma unroll
            for (int k = 0; k < kTiles; ++k)
                if (k == 0 || r + 16 * k < it.row1) compute_tile(r + 16 * k, t[k]);
        };
        while (r0 + kStep < it.row1) {          // steps r0 and r0 + kStep both hold rows
            load_step(r0 + kStep, tb);
            compute_step(r0, ta);
            load_step(r0 + 2 * kStep, ta);
            compute_step(r0 + kStep, tb);
            r0 += 2 * kStep;
            progress(2 * kTiles);
        }
        if (r0 < it.row1) compute_step(r0, ta);

        // ---- the piece's partial: (max, sum) and the f64 accumulators per head ----
        if (since_flush) flush();
#pragma unroll
        for (int hb = 0; hb < NB; ++hb) {
            double lt = l[hb];
#pragma unroll
            for (int msk = 1; msk < 16; msk <<= 1) lt += shfl_xor_f64(lt, msk);
            const int h = 4 * hb + hq;
            if (n == 0 && h < HPK) {
                const size_t ix = (size_t)it.slot * HPK + h;
                a.ws_ml[ix * 2] = m[hb];
                a.ws_ml[ix * 2 + 1] = (float)lt;
            }
        }
#pragma unroll
        for (int i = 0; i < kOwn; ++i) {
            const int e = kOwn * ri + i;
            a.ws_acc[((size_t)it.slot * HPK + e / kVDim) * kHD + kVDim * seg + e % kVDim] = (float)cell(i);
        }
    });
}

// ---------------------------------------------------------------------------
// Combine: per (sequence, Q head), merge the partials of the segment with
// the same rescaling as the fold ([P3] fold: accumulators are rescaled by
// exp(old max - new max)), divide, and apply the V column field (q8 only).
// Empty partials (max -inf) weigh nothing.  Q heads of dead groups, and
// sequences with no rows, get zeros.  When the (sequence, head) grid is
// small (R-SWA: 10 heads), a head's 128 channels are split over up to eight
// blocks, so that more compute units share the read of its partials; a block
// then has sub-groups of lpg = 32 / chunks lanes (a float4 of channels
// each), as many as its partial count asks for (at most 512 threads).  A
// sub-group takes every ngroups-th partial, issuing the loads of up to 8 at
// once and folding them with a running max.  The sub-groups of a wave then
// merge by a butterfly over lanes lpg, 2 lpg, .. apart, and the block's
// waves (at most 8) merge in LDS.  Blocks are whole waves: sub-groups past
// the partial count hold empty states (max -inf, sum 0).
// ---------------------------------------------------------------------------
#ifndef KVQ_COMBINE_THREADS
#define KVQ_COMBINE_THREADS 512
#endif
#ifndef KVQ_COMBINE_BATCH
#define KVQ_COMBINE_BATCH 8
#endif
constexpr int kCombineThreads = KVQ_COMBINE_THREADS;
constexpr int kCombineBatch = KVQ_COMBINE_BATCH;

// Channel chunks per head for a grid of `blocks` (sequence, head) pairs.
// (R-SWA, 10 pairs: 8 chunks took the int8 step from 23.3 to 22.8 us.)
inline int combine_chunks(int blocks) { return blocks >= 256 ? 1 : blocks >= 128 ? 2 : blocks >= 64 ? 4 : 8; }

// Folds the nch partials at ml / acc (strides mstride / astride floats),
// channels ch0 .. ch0 + 4 lpg - 1, with a sink logit zs in log2 units (-inf:
// none) and leaves, for tid < lpg, the normalised channels ch0 + 4 tid ..
// + 3 in *res.  Block-wide: every thread of the block calls it.
__device__ __forceinline__ bool combine_partials(const float* ml, const float* acc, size_t mstride, size_t astride,
                                                 int nch, float zs, int lpg, int ch0, float4* res) {
    __shared__ float4 sm_acc[kCombineThreads / 64][32];
    __shared__ float sm_m[kCombineThreads / 64], sm_l[kCombineThreads / 64];
    const int tid = threadIdx.x;
    const int sg = tid / lpg, lane = tid - sg * lpg;
    const int ngroups = (int)blockDim.x / lpg;
    const int wave = tid >> 6, nwaves = (int)blockDim.x >> 6;

    float M = -INFINITY, L = 0.0f;
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c0 = sg; c0 < nch; c0 += ngroups * kCombineBatch) {
        float mv[kCombineBatch], lv[kCombineBatch];
        float4 xv[kCombineBatch];
#pragma unroll
        for (int k = 0; k < kCombineBatch; ++k) {
            const int c = c0 + k * ngroups;
            const bool ok = c < nch;
            const float2 x = ok ? *(const float2*)(ml + c * mstride) : make_float2(-INFINITY, 0.0f);
            mv[k] = x.x;
            lv[k] = x.y;
            xv[k] = ok ? *(const float4*)(acc + c * astride + ch0 + 4 * lane) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        float Mn = M;
#pragma unroll
        for (int k = 0; k < kCombineBatch; ++k) Mn = fmaxf(Mn, mv[k]);
        const float r = M == Mn ? 1.0f : fast_exp2(M - Mn);   // 0 while M is still -inf
        L *= r;
        A.x *= r;
        A.y *= r;
        A.z *= r;
        A.w *= r;
#pragma unroll
        for (int k = 0; k < kCombineBatch; ++k) {
            const float e = mv[k] == -INFINITY ? 0.0f : fast_exp2(mv[k] - Mn);   // empty partials
            L = fmaf(e, lv[k], L);
            A.x = fmaf(e, xv[k].x, A.x);
            A.y = fmaf(e, xv[k].y, A.y);
            A.z = fmaf(e, xv[k].z, A.z);
            A.w = fmaf(e, xv[k].w, A.w);
        }
        M = Mn;
    }
    // the wave's sub-groups: butterfly over lanes lpg, 2 lpg, .. apart
    for (int msk = lpg; msk < 64; msk <<= 1) {
        const float Mo = __shfl_xor(M, msk, 64), Lo = __shfl_xor(L, msk, 64);
        const float4 Ao = make_float4(__shfl_xor(A.x, msk, 64), __shfl_xor(A.y, msk, 64),
                                      __shfl_xor(A.z, msk, 64), __shfl_xor(A.w, msk, 64));
        const float Mn = fmaxf(M, Mo);
        const float e0 = M == -INFINITY ? 0.0f : fast_exp2(M - Mn);
        const float e1 = Mo == -INFINITY ? 0.0f : fast_exp2(Mo - Mn);
        L = L * e0 + Lo * e1;
        A.x = A.x * e0 + Ao.x * e1;
        A.y = A.y * e0 + Ao.y * e1;
        A.z = A.z * e0 + Ao.z * e1;
        A.w = A.w * e0 + Ao.w * e1;
        M = Mn;
    }
    if ((tid & 63) < lpg) {
        sm_acc[wave][tid & 63] = A;
        if ((tid & 63) == 0) {
            sm_m[wave] = M;
            sm_l[wave] = L;
        }
    }
    __syncthreads();
    if (tid >= lpg) return false;
    // the sink logit enters the running max and the normaliser, with no V
    // row ([P2] attend_group_upto)
    float Mt = zs;
    for (int k = 0; k < nwaves; ++k) Mt = fmaxf(Mt, sm_m[k]);
    float Lt = zs == -INFINITY ? 0.0f : fast_exp2(zs - Mt);
    float4 At = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < nwaves; ++k) {
        const float e = sm_m[k] == -INFINITY ? 0.0f : fast_exp2(sm_m[k] - Mt);   // waves without rows
        const float4 x = sm_acc[k][tid];
        Lt = fmaf(e, sm_l[k], Lt);
        At.x = fmaf(e, x.x, At.x);
        At.y = fmaf(e, x.y, At.y);
        At.z = fmaf(e, x.z, At.z);
        At.w = fmaf(e, x.w, At.w);
    }
    const float inv = 1.0f / Lt;
    *res = make_float4(At.x * inv, At.y * inv, At.z * inv, At.w * inv);
    return true;
}

// Block (Q head h x channel chunk, sequence j); chunks = gridDim.x / n_q_heads.
template <bool kQ8>
__global__ __launch_bounds__(kCombineThreads) void k_combine(const DecodeArgs a) {
    const int chunks = (int)gridDim.x / a.n_q_heads;
    const int h = blockIdx.x / chunks, ck = blockIdx.x - h * chunks;
    const int lpg = 32 / chunks, ch0 = 4 * lpg * ck;
    const int j = blockIdx.y, tid = threadIdx.x;
    const int b = a.seq0 + j;
    const int g = h / a.hpk, hh = h - g * a.hpk;
    const int gl = arg_byte(a.live_slot, g);
    float* o = a.out + ((size_t)b * a.n_q_heads + h) * kHD + ch0;
    const int nt = a.ntile[j];
    if (gl < 0 || nt == 0) {
        if (tid < lpg) *(float4*)(o + 4 * tid) = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }
    // slots of the segment: its first..last share + segment index
    const int sb = a.tile_base[j] + gl * nt;
    const int first = tile_owner(sb, a.n_tiles, a.n_shares);
    const int nch = tile_owner(sb + nt - 1, a.n_tiles, a.n_shares) - first + 1;
    const size_t it0 = (size_t)first + (size_t)j * a.n_live + gl;
    const float zs = a.sinks ? (float)((double)a.sinks[h] * 1.4426950408889634) : -INFINITY;
    // the V column field is loaded before the partials, so that its latency
    // overlaps theirs
    const bool frz = kQ8 && arg_byte(a.frozen, j);
    float4 vc = make_float4(1.f, 1.f, 1.f, 1.f);
    if (frz && tid < lpg) vc = *(const float4*)(a.vcol + ((size_t)b * a.n_live + gl) * kHD + ch0 + 4 * tid);
    float4 rr;
    if (!combine_partials(a.ws_ml + (it0 * a.hpk + hh) * 2, a.ws_acc + (it0 * a.hpk + hh) * kHD,
                          (size_t)a.hpk * 2, (size_t)a.hpk * kHD, nch, zs, lpg, ch0, &rr))
        return;
    if (frz) {
        rr.x *= vc.x;
        rr.y *= vc.y;
        rr.z *= vc.z;
        rr.w *= vc.w;
    }
    *(float4*)(o + 4 * tid) = rr;
}

// ---------------------------------------------------------------------------
// K-token R-SWA verify ([P3] verify_attention): every draft query attends
// the reference rows, the ring as it would stand after the drafts up to its
// own were written, and those drafts; nothing is written.  Up to 16 queries
// per KV head (n_draft x hpk) share each K and V row read, which makes the
// score and value passes dense contractions on the matrix cores
// (v_mfma_f32_16x16x4f32, f32 in and out):
//   scores  S^T[16 rows x 16 queries] = K[16 x 128] Q^T: A = K (lane l: row
//           l % 16, channels 16 u + 4 (l / 16) + e, u < 8, e < 4, so the four
//           lanes of a row read 64 contiguous bytes per load), B = Q^T (lane
//           l: query l % 16, the same channels), 32 steps; lane l receives the
//           scores of query l % 16 for rows 4 (l / 16) + r, r < 4;
//   values  (P V)^T[channels x queries] = V^T P^T per 16-channel block cb:
//           step s takes row 4 (l / 16) + s from each lane, so the B operand
//           is the lane's own weight p[s] and the A operand is V[row][c] with
//           c = 4 (l % 16) + (cb & 3) + 64 (cb >> 2) (16 lanes read 256
//           contiguous bytes); lane l accumulates query l % 16's channels
//           16 (l / 16) + 4 r + (cb & 3) + 64 (cb >> 2) -- one query per lane,
//           so the online-softmax rescale is per lane.
// Visibility of row p to draft query i (the ring after i + 1 more writes):
// reference rows always; a ring slot unless it is among the e_i = max(0,
// ring_len + i + 1 - 128) oldest live slots; draft row d iff d <= i.
// ---------------------------------------------------------------------------
// kShared: the shared-reference decode -- the "drafts" are streams sharing
// the sequence's reference rows [0, prefill); stream s owns the ring rows
// prefill + 128 s .. + 127.  The row space is the reference, the S rings,
// then the S step rows (read from kd / vd, like drafts): stream s sees the
// reference, its ring slots that were live before this step except the one
// the step overwrites, and its own step row.  The wave whose share holds
// step row s also stores it into stream s's ring.
// Occupancy: the verify (kShared false) runs one wave per SIMD and may use
// the whole register file (up to 512 registers); the shared decode stays at
// two waves' worth (256).  Measured on MI355X, 32k R-SWA reference, 8
// drafts: 65.2 -> 64.0 us per call.  The shared decode was slower with the
// same setting (78.4 against 75.0 us, both measured with a variant of its
// step-row copy).  More tiles in flight did not pay for the verify: 3 tiles
// 65.4 us, 4 tiles 68.3 us.
template <bool kShared>
__global__ __launch_bounds__(256, kShared ? 2 : 1) void k_verify_f32(const VerifyArgs a) {
    const int w = share_index();
    if (w >= a.n_shares) return;
    const int lane = threadIdx.x & 63;
    const int qi = lane & 15, kb = lane >> 4;
    for_each_piece(a, w, [&](const Piece& it) {
        if (it.row0 >= it.row1) {
            // only padding tiles past the segment's rows (see launch_verify_f32):
            // an empty partial
            if (qi < a.nq) {
                const size_t ix = (size_t)it.slot * a.nq + qi;
                if (kb == 0) {
                    a.ws_ml[ix * 2] = -INFINITY;
                    a.ws_ml[ix * 2 + 1] = 0.0f;
                }
                float* dst = a.ws_acc + ix * kHD + 16 * kb;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    *(float4*)(dst + 4 * r) = make_float4(0.f, 0.f, 0.f, 0.f);
                    *(float4*)(dst + 64 + 4 * r) = make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
            return;
        }
        const int j = it.j;
        const int pre = a.prefill[j];
        const int L = kShared ? pre + KVQ_RING_WINDOW * a.n_draft       // reference + rings; step rows follow
                              : pre + a.ring_len[j];                     // cache rows; drafts follow
        const float* K = a.k + it.hrow * kHD;
        const float* V = a.v + it.hrow * kHD;
        const size_t dstride = (size_t)a.n_kv_heads * kHD;
        const size_t ob = kShared ? 0 : (size_t)it.b;                    // batch index of q / k_draft / out
        const float* KD = a.kd + (ob * a.n_draft * a.n_kv_heads + it.g) * kHD;
        const float* VD = a.vd + (ob * a.n_draft * a.n_kv_heads + it.g) * kHD;
        auto row_ptr = [&](const float* C, const float* D, int p) {
            return p < L ? C + (size_t)p * kHD : D + (size_t)(p - L) * dstride;
        };
        if constexpr (kShared) {
            // [P3] write_decode_step of each stream whose step row is in this
            // piece: lane l copies stream l / 4's channels 32 (l % 4) .., all
            // its loads issued before its stores.  Named registers: as two
            // float4[8] arrays the copy was kept in scratch memory (272 bytes
            // per lane), at the same speed.
            const int s = lane >> 2, c0 = 32 * (lane & 3);
            if (s < a.n_draft && L + s >= it.row0 && L + s < it.row1) {
                const size_t wr = it.hrow + (size_t)a.swrow[s];
                const float4* ksrc = (const float4*)(KD + s * dstride + c0);
                const float4* vsrc = (const float4*)(VD + s * dstride + c0);
                float4* kdst = (float4*)(a.k_store + wr * kHD + c0);
                float4* vdst = (float4*)(a.v_store + wr * kHD + c0);
                const float4 k0 = ksrc[0], k1 = ksrc[1], k2 = ksrc[2], k3 = ksrc[3];
                const float4 k4 = ksrc[4], k5 = ksrc[5], k6 = ksrc[6], k7 = ksrc[7];
                const float4 v0 = vsrc[0], v1 = vsrc[1], v2 = vsrc[2], v3 = vsrc[3];
                const float4 v4 = vsrc[4], v5 = vsrc[5], v6 = vsrc[6], v7 = vsrc[7];
                kdst[0] = k0; kdst[1] = k1; kdst[2] = k2; kdst[3] = k3;
                kdst[4] = k4; kdst[5] = k5; kdst[6] = k6; kdst[7] = k7;
                vdst[0] = v0; vdst[1] = v1; vdst[2] = v2; vdst[3] = v3;
                vdst[4] = v4; vdst[5] = v5; vdst[6] = v6; vdst[7] = v7;
            }
        }
        // this lane's query (MFMA column): draft (stream) di, head hh of the group
        const bool qvalid = qi < a.nq;
        const int di = qvalid ? qi / a.hpk : 0, hh = qvalid ? qi - di * a.hpk : 0;
        float qb[32];
        {
            const float* qp = a.q + ((ob * a.n_draft + di) * a.n_q_heads + it.g * a.hpk + hh) * kHD + 4 * kb;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float4 x = qvalid ? *(const float4*)(qp + 16 * t) : make_float4(0.f, 0.f, 0.f, 0.f);
                qb[4 * t + 0] = x.x * kQScale;
                qb[4 * t + 1] = x.y * kQScale;
                qb[4 * t + 2] = x.z * kQScale;
                qb[4 * t + 3] = x.w * kQScale;
            }
        }
        const int rl = a.ring_len[j], old = a.ring_oldest[j];
        const int evict = max(0, rl + di + 1 - KVQ_RING_WINDOW);
        const int live = kShared ? a.sring[di] : 0;                             // ring slots live before the step
        const int wslot = kShared ? a.swrow[di] - pre - KVQ_RING_WINDOW * di : 0; // the slot it overwrites
        auto visible = [&](int p) {
            if (p < pre) return true;
            if constexpr (kShared) {
                if (p >= L) return p - L == di;
                const int slot = (p - pre) & (KVQ_RING_WINDOW - 1);
                return ((p - pre) >> 7) == di && slot < live && slot != wslot;
            } else {
                if (p < L) return ((p - pre - old + KVQ_RING_WINDOW) & (KVQ_RING_WINDOW - 1)) >= evict;
                return p - L <= di;
            }
        };

        struct Tile {
            float4 kt[8];      // K row r0 + qi, channels 16 u + 4 kb ..
            float4 vt[4][2];   // V rows r0 + 4 kb + s, channels 4 qi .. and 64 + 4 qi ..
        };
        auto load_k = [&](int r0, Tile& t) {
            const float* kr = row_ptr(K, KD, min(r0 + qi, it.row1 - 1)) + 4 * kb;
#pragma unroll
            for (int u = 0; u < 8; ++u) t.kt[u] = ld_stream(kr + 16 * u);
        };
        auto load_v = [&](int r0, Tile& t) {
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const float* vr = row_ptr(V, VD, min(r0 + 4 * kb + s2, it.row1 - 1)) + 4 * qi;
                t.vt[s2][0] = ld_stream(vr);
                t.vt[s2][1] = ld_stream(vr + 64);
            }
        };
        float m = -INFINITY, l = 0.0f;
        v4f acc[8];
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) acc[cb] = v4f{0.f, 0.f, 0.f, 0.f};
        // Tile t's arithmetic; with kReload, the tile of row rn is then loaded
        // into t, its K rows as soon as the score MFMAs have read t's (so
        // they are in flight during the rest of this tile and the next one),
        // its V rows after the value MFMAs.
        auto compute_tile = [&](int r0, Tile& t, int rn, auto reload) {
            constexpr bool kReload = decltype(reload)::value;
            v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                c = __builtin_amdgcn_mfma_f32_16x16x4f32(t.kt[u].x, qb[4 * u + 0], c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x4f32(t.kt[u].y, qb[4 * u + 1], c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x4f32(t.kt[u].z, qb[4 * u + 2], c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x4f32(t.kt[u].w, qb[4 * u + 3], c, 0, 0, 0);
            }
            if constexpr (kReload) load_k(rn, t);
            float sc[4];
            float tmax = -INFINITY;
            if (kShared && r0 >= pre && r0 + kTileRows <= min(L, it.row1) &&
                ((r0 - pre) >> 7) == ((r0 + kTileRows - 1 - pre) >> 7)) {
                // a whole tile of stream ts's ring (wave-uniform): only that
                // stream's queries see it, each of its live slots but the one
                // this step overwrites (on MI355X, 32k reference and 16
                // streams, 70.6 -> 68.3 us per call against the general test)
                const int ts = (r0 - pre) >> 7;
                const int s0 = ((r0 - pre) & (KVQ_RING_WINDOW - 1)) + 4 * kb;
                const bool mine = qvalid && di == ts;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sc[r] = (mine && s0 + r < live && s0 + r != wslot) ? c[r] : -INFINITY;
                    tmax = fmaxf(tmax, sc[r]);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int p = r0 + 4 * kb + r;
                    sc[r] = (qvalid && p < it.row1 && visible(p)) ? c[r] : -INFINITY;
                    tmax = fmaxf(tmax, sc[r]);
                }
            }
            tmax = max_rows(tmax);
            const float mnew = fmaxf(m, tmax);
            const float alpha = mnew == -INFINITY ? 1.0f : fast_exp2(m - mnew);
            float pw[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) pw[r] = sc[r] == -INFINITY ? 0.0f : fast_exp2(sc[r] - mnew);
            l = l * alpha + ((pw[0] + pw[1]) + (pw[2] + pw[3]));
            m = mnew;
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) acc[cb] *= alpha;
            // Shared decode: a ring row that no stream may read -- a slot never
            // written since the prefill (its memory may hold anything, NaN
            // included), or the slot this step overwrites -- enters the value
            // product as zeros, so that a zero weight times it stays zero.  A
            // tile that reaches into the rings (wave-uniform) spans at most two
            // streams' rings; their cursors come through scalar loads (per-lane
            // loads of them would wait behind the prefetched tile's loads).
            bool ok[4] = {true, true, true, true};
            if (kShared && r0 + kTileRows > pre && r0 < L) {
                const int s_lo = __builtin_amdgcn_readfirstlane(max(0, (r0 - pre) >> 7));
                const int s_hi = __builtin_amdgcn_readfirstlane(min(a.n_draft - 1, (r0 + kTileRows - 1 - pre) >> 7));
                const int live_lo = a.sring[s_lo], live_hi = a.sring[s_hi];
                const int over_lo = a.swrow[s_lo] - pre - KVQ_RING_WINDOW * s_lo;
                const int over_hi = a.swrow[s_hi] - pre - KVQ_RING_WINDOW * s_hi;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                    const int p = r0 + 4 * kb + s2;
                    const int rs = (p - pre) >> 7, slot = (p - pre) & (KVQ_RING_WINDOW - 1);
                    const int lv = rs == s_lo ? live_lo : live_hi, ov = rs == s_lo ? over_lo : over_hi;
                    ok[s2] = p < pre || p >= L || (slot < lv && slot != ov);
                }
            }
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                float vv[8] = {t.vt[s2][0].x, t.vt[s2][0].y, t.vt[s2][0].z, t.vt[s2][0].w,
                               t.vt[s2][1].x, t.vt[s2][1].y, t.vt[s2][1].z, t.vt[s2][1].w};
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) vv[cb] = ok[s2] ? vv[cb] : 0.0f;
#pragma unroll
                for (int cb = 0; cb < 8; ++cb)
                    acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv[cb], pw[s2], acc[cb], 0, 0, 0);
            }
            if constexpr (kReload) load_v(rn, t);
        };
        // Two tiles in registers, each reloaded from inside its own arithmetic;
        // the loop exits only at its head (as in k_decode_q8: a break between
        // the halves makes the compiler drain every load there).  Loads past
        // the piece's last row read that row again.  Measured on MI355X, 32k
        // R-SWA reference, against reloading a tile after its arithmetic: verify
        // (8 drafts) 64.1 -> 62.2 us, shared decode (16 streams) 68.4 -> 66.3 us
        // per call; the same loads with no arithmetic take 58.8 us.  Three
        // tiles in registers: verify 63.1 us, and the shared decode spills.
        using Reload = std::true_type;
        using Last = std::false_type;
        int r0 = it.row0;
        Tile ta, tb;
        load_k(r0, ta);
        load_v(r0, ta);
        load_k(r0 + kTileRows, tb);
        load_v(r0 + kTileRows, tb);
        while (r0 + 2 * kTileRows < it.row1) {
            compute_tile(r0, ta, r0 + 2 * kTileRows, Reload{});
            compute_tile(r0 + kTileRows, tb, r0 + 3 * kTileRows, Reload{});
            r0 += 2 * kTileRows;
        }
        compute_tile(r0, ta, 0, Last{});
        if (r0 + kTileRows < it.row1) compute_tile(r0 + kTileRows, tb, 0, Last{});
        // the piece's partial for each valid query
        const float lt = sum_rows(l);
        if (qvalid) {
            const size_t ix = (size_t)it.slot * a.nq + qi;
            if (kb == 0) {
                a.ws_ml[ix * 2] = m;
                a.ws_ml[ix * 2 + 1] = lt;
            }
            float* dst = a.ws_acc + ix * kHD + 16 * kb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                *(float4*)(dst + 4 * r) = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
                *(float4*)(dst + 64 + 4 * r) = make_float4(acc[4][r], acc[5][r], acc[6][r], acc[7][r]);
            }
        }
    });
}

// ---------------------------------------------------------------------------
// The query-batched kernel on the per-row int8 kind: [P3] verify_attention and
// batched_decode_attention go through decode_attention, which with the int8
// mirror is decode_attention_int8 -- every query quantised per head
// (quantize_row_i8), exact i32 dots with the K codes scaled by qscale and the
// row's K scale, V codes dequantised by the row's V scale.  Up to 16 queries
// per KV head share each row read:
//   scores  v_mfma_i32_16x16x64_i8, A = K codes (lane l: row l % 16 of the
//           tile, 16 channels at 16 (l / 16) + 64 sp), B = the 16 queries'
//           codes (lane l: query l % 16, the same channels), one MFMA per
//           64-channel span; lane l receives rows 4 (l / 16) + r of query
//           l % 16, scaled in f64;
//   values  (P V)^T = V^T P^T on v_mfma_f32_16x16x32_bf16, one pair per
//           8-channel block cb (channels 8 m + cb, m = l % 16): lane l's eight
//           K slots are its four rows 4 (l / 16) + r, twice.  A = those rows'
//           V codes (exact in bf16, each twice); B = the lane's own query's
//           weights times the rows' V scales, split exactly into three bf16
//           parts (hi, mid in the first MFMA's slots, lo and zeros in the
//           second's), so the f32 accumulators receive the f32 weights' full
//           products.  Lane l accumulates query l % 16's channels
//           8 (4 (l / 16) + r) + cb.
// The running max is lazy (moved only when a tile's max exceeds it by more
// than kLazy), so the 32 accumulators are rarely rescaled.
// Rows past the cache's ("trailing rows": the verify's drafts, the shared
// decode's step rows, one per stream) are quantised with quantize_row_i8 by
// each wave whose share holds them, into its LDS, at the start of the piece;
// in the shared decode the wave also stores stream s's quantised step row in
// the stream's ring slot ([P3] write_decode_step), where no other wave reads
// it during this call (the slot is masked for stream s, invisible to the
// others).
// Verify: query i sees the reference, the ring slots that survive drafts
// 0..i, and drafts 0..i.  Shared decode: stream s sees the reference, its
// ring slots live before the step except the one the step overwrites, and its
// own step row.
// ---------------------------------------------------------------------------
#ifndef KVQ_VI8_FAST_SHARED
#define KVQ_VI8_FAST_SHARED 1
#endif
// Tiles a wave keeps in flight (registers) while it computes: one share per
// SIMD, so a wave has the SIMD's registers to itself and its loads, not its
// occupancy, hide the memory latency.
#ifndef KVQ_VI8_DEPTH
#define KVQ_VI8_DEPTH 4
#endif
// Two waves' worth of registers (256).  Measured on MI355X, 32k R-SWA
// reference: with the whole register file (one wave per SIMD, up to 512)
// the verify took 27.0 against 26.6 us and the shared decode 30.1 against
// 29.2 us; 6 tiles in flight there 27.9 / 31.2 us.
template <bool kShared>
__global__ __launch_bounds__(256, 2) void k_verify_i8(const VerifyArgs a) {
    constexpr int D = KVQ_VI8_DEPTH;
    // trailing rows of the piece: K / V codes and scales
    __shared__ __attribute__((aligned(16))) int8_t sm_tq[kWaves][2][kVerifyMaxQ][kHD];
    __shared__ float sm_ts[kWaves][2][kVerifyMaxQ];
    const int w = share_index();
    if (w >= a.n_shares) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int qi = lane & 15, kb = lane >> 4;
    for_each_piece(a, w, [&](const Piece& it) {
        if (it.row0 >= it.row1) {
            // only padding tiles past the segment's rows (see launch_verify_i8):
            // an empty partial
            if (qi < a.nq) {
                const size_t ix = (size_t)it.slot * a.nq + qi;
                if (kb == 0) {
                    a.ws_ml[ix * 2] = -INFINITY;
                    a.ws_ml[ix * 2 + 1] = 0.0f;
                }
                float* dst = a.ws_acc + ix * kHD + 32 * kb;
#pragma unroll
                for (int r = 0; r < 8; ++r) *(float4*)(dst + 4 * r) = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            return;
        }
        const int j = it.j;
        const int pre = a.prefill[j];
        const int L = kShared ? pre + KVQ_RING_WINDOW * a.n_draft : pre + a.ring_len[j];   // cache rows
        const size_t ob = kShared ? 0 : (size_t)it.b;
        const int8_t* KQ = a.kq + it.hidx * kq_rows(a.capacity) * kHD;   // tile-major K codes
        const float* KS = a.ks + it.hrow;
        const int8_t* VQ = a.vq + it.hrow * kHD;
        const float* VS = a.vs + it.hrow;

        // this lane's query (B column): draft / stream di, head hh of the
        // group; its loads go out first, ahead of the trailing rows' and the
        // tiles', so that its quantisation waits for it alone
        const bool qvalid = qi < a.nq;
        const int di = qvalid ? qi / a.hpk : 0, hh = qvalid ? qi - di * a.hpk : 0;
        float4 qv[2][4];
        {
            const float* qp = a.q + ((ob * a.n_draft + di) * a.n_q_heads + it.g * a.hpk + hh) * kHD + 16 * kb;
#pragma unroll
            for (int sp = 0; sp < 2; ++sp)
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4)
                    qv[sp][t4] = qvalid ? *(const float4*)(qp + 64 * sp + 4 * t4) : make_float4(0.f, 0.f, 0.f, 0.f);
        }

        // ---- trailing rows [t0, t1) of this piece, quantised into LDS ----
        // Lane l takes row t0 + l / 4 and the 32 channels 32 (l % 4) .. of its
        // K and V (all loads issued at once); a row's scale is the max over its
        // four lanes.  The loads go out before the first tile's, the
        // arithmetic after them.
        const int t0 = max(it.row0, L) - L, t1 = it.row1 - L;
        const int tr = t0 + (lane >> 2), tc = 32 * (lane & 3);
        const bool tlane = tr < t1;
        float4 xk[8], xv[8];
        if (t1 > 0) {
            const size_t dstride = (size_t)a.n_kv_heads * kHD;
            const size_t off = (ob * a.n_draft * a.n_kv_heads + it.g) * kHD + (size_t)(tlane ? tr : t0) * dstride + tc;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                xk[u] = *(const float4*)(a.kd + off + 4 * u);
                xv[u] = *(const float4*)(a.vd + off + 4 * u);
            }
        }
        auto quantise_trailing = [&]() {
            float ak = 0.0f, av = 0.0f;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                ak = fmaxf(ak, fmaxf(fmaxf(fabsf(xk[u].x), fabsf(xk[u].y)), fmaxf(fabsf(xk[u].z), fabsf(xk[u].w))));
                av = fmaxf(av, fmaxf(fmaxf(fabsf(xv[u].x), fabsf(xv[u].y)), fmaxf(fabsf(xv[u].z), fabsf(xv[u].w))));
            }
            ak = fmaxf(ak, __shfl_xor(ak, 1, 64));
            ak = fmaxf(ak, __shfl_xor(ak, 2, 64));
            av = fmaxf(av, __shfl_xor(av, 1, 64));
            av = fmaxf(av, __shfl_xor(av, 2, 64));
            const float sk = ak > 0.0f ? __fdiv_rn(ak, 127.0f) : 1.0f;
            const float sv = av > 0.0f ? __fdiv_rn(av, 127.0f) : 1.0f;
            const float ik = __fdiv_rn(1.0f, sk), iv = __fdiv_rn(1.0f, sv);
            auto code = [](float x, float sc, float inv) { return (int)fminf(fmaxf(rint_div(x, sc, inv), -127.0f), 127.0f) & 0xff; };
            uint32_t ck[8], cv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                ck[u] = code(xk[u].x, sk, ik) | (code(xk[u].y, sk, ik) << 8) | (code(xk[u].z, sk, ik) << 16) |
                        (code(xk[u].w, sk, ik) << 24);
                cv[u] = code(xv[u].x, sv, iv) | (code(xv[u].y, sv, iv) << 8) | (code(xv[u].z, sv, iv) << 16) |
                        (code(xv[u].w, sv, iv) << 24);
            }
            if (tlane) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    *(uint4*)(&sm_tq[wave][0][tr][tc + 16 * h]) = make_uint4(ck[4 * h], ck[4 * h + 1], ck[4 * h + 2], ck[4 * h + 3]);
                    *(uint4*)(&sm_tq[wave][1][tr][tc + 16 * h]) = make_uint4(cv[4 * h], cv[4 * h + 1], cv[4 * h + 2], cv[4 * h + 3]);
                }
                if ((lane & 3) == 0) {
                    sm_ts[wave][0][tr] = sk;
                    sm_ts[wave][1][tr] = sv;
                }
                if constexpr (kShared) {
                    // [P3] write_decode_step: stream tr's step row into its ring slot
                    const int row = a.swrow[tr];
                    int8_t* kdst = a.kq + it.hidx * kq_rows(a.capacity) * kHD;
                    int8_t* vdst = a.vq + (it.hrow + row) * kHD + tc;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        *(uint4*)(kdst + kq_offset(row, tc + 16 * h)) = make_uint4(ck[4 * h], ck[4 * h + 1], ck[4 * h + 2], ck[4 * h + 3]);
                        *(uint4*)(vdst + 16 * h) = make_uint4(cv[4 * h], cv[4 * h + 1], cv[4 * h + 2], cv[4 * h + 3]);
                    }
                    if ((lane & 3) == 0) {
                        a.ks[it.hrow + row] = sk;
                        a.vs[it.hrow + row] = sv;
                    }
                }
            }
            wave_lds_sync();
        };
        struct Tile {
            uint4 kc[2];       // K codes of row r0 + qi, spans 0 and 1
            float ks[4];       // K scales of rows r0 + 4 kb + r
            uint2 vc[4];       // V codes of rows r0 + 4 kb + s, channels 8 qi ..
            float vs[4];
        };
        auto load_tile = [&](int r0, Tile& t) {
            if ((!kShared || KVQ_VI8_FAST_SHARED) && min(r0 + kTileRows - 1, it.row1 - 1) < L) {
                // the whole tile in the cache (wave-uniform): no per-row choice
                // of source, 32-bit offsets from the block's scalar base
                const uint32_t pk = (uint32_t)min(r0 + qi, it.row1 - 1);
                t.kc[0] = ld_stream(KQ + kq_offset((int)pk, 16 * kb));
                t.kc[1] = ld_stream(KQ + kq_offset((int)pk, 64 + 16 * kb));
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t p = (uint32_t)min(r0 + 4 * kb + r, it.row1 - 1);
                    t.ks[r] = KS[p];                   // row scales: plain loads, as in k_decode_q8
                    ld_v(VQ + (p * kHD + 8 * qi), t.vc[r]);
                    t.vs[r] = VS[p];
                }
                return;
            }
            const int pk = min(r0 + qi, it.row1 - 1);
            if (pk < L) {
                t.kc[0] = ld_stream(KQ + kq_offset(pk, 16 * kb));
                t.kc[1] = ld_stream(KQ + kq_offset(pk, 64 + 16 * kb));
            } else {                                     // a trailing row, from LDS
                t.kc[0] = *(const uint4*)(&sm_tq[wave][0][pk - L][16 * kb]);
                t.kc[1] = *(const uint4*)(&sm_tq[wave][0][pk - L][64 + 16 * kb]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int p = min(r0 + 4 * kb + r, it.row1 - 1);
                if (p < L) {
                    t.ks[r] = KS[p];
                    ld_v(VQ + (size_t)p * kHD + 8 * qi, t.vc[r]);
                    t.vs[r] = VS[p];
                } else {
                    t.ks[r] = sm_ts[wave][0][p - L];
                    t.vc[r] = *(const uint2*)(&sm_tq[wave][1][p - L][8 * qi]);
                    t.vs[r] = sm_ts[wave][1][p - L];
                }
            }
        };
        // a whole tile of cache rows (no per-row clamp or choice of source):
        // the lane's four consecutive rows' scales in one (dword-aligned) load
        // per buffer
        auto load_whole_k = [&](int r0, Tile& t) {
            const uint32_t pk = (uint32_t)(r0 + qi), p = (uint32_t)(r0 + 4 * kb);
            t.kc[0] = ld_stream(KQ + kq_offset((int)pk, 16 * kb));
            t.kc[1] = ld_stream(KQ + kq_offset((int)pk, 64 + 16 * kb));
            const float4 k4 = *(const float4*)(KS + p);
            t.ks[0] = k4.x, t.ks[1] = k4.y, t.ks[2] = k4.z, t.ks[3] = k4.w;
        };
        auto load_whole_v = [&](int r0, Tile& t) {
            const uint32_t p = (uint32_t)(r0 + 4 * kb);
#pragma unroll
            for (int r = 0; r < 4; ++r) ld_v(VQ + ((p + r) * kHD + 8 * qi), t.vc[r]);
            const float4 v4 = *(const float4*)(VS + p);
            t.vs[0] = v4.x, t.vs[1] = v4.y, t.vs[2] = v4.z, t.vs[3] = v4.w;
        };
        auto load_whole = [&](int r0, Tile& t) {
            load_whole_k(r0, t);
            load_whole_v(r0, t);
        };
        // either loader, as the tile asks
        auto load_any = [&](int r0, Tile& t) {
            if (r0 + kTileRows <= min(L, it.row1))
                load_whole(r0, t);
            else
                load_tile(r0, t);
        };
        // The first D tiles' loads go out before the trailing rows' arithmetic
        // and the query set-up (a piece is never empty).  In the verify, when
        // the piece starts with whole tiles of cache rows, D whole-tile loads
        // (8 loads each) go out unconditionally (past the last whole tile:
        // that one again), so the waits below count exactly the loads in
        // flight, and stay within what the wave's counter tracks (63); the
        // tiles they did not cover (partial, or reading trailing rows from
        // LDS) load after the trailing rows are quantised.  (The shared
        // decode keeps the conditional loads: with the unconditional ones its
        // registers spill and its last wave per head slows down.)
        const int ntl = (it.row1 - it.row0 + kTileRows - 1) / kTileRows;
        const int nwhole = (min(L, it.row1) - it.row0) / kTileRows;
        auto in_cache = [&](int r0) { return min(r0 + kTileRows - 1, it.row1 - 1) < L; };
        Tile tl[D];
        if (!kShared && nwhole > 0) {
#pragma unroll
            for (int i = 0; i < D; ++i) load_whole(it.row0 + kTileRows * min(i, nwhole - 1), tl[i]);
            if (t1 > 0) quantise_trailing();
#pragma unroll
            for (int i = 0; i < D; ++i)
                if (i >= nwhole && i < ntl) load_tile(it.row0 + kTileRows * i, tl[i]);
        } else {
#pragma unroll
            for (int i = 0; i < D; ++i)
                if (i < ntl && in_cache(it.row0 + kTileRows * i)) load_tile(it.row0 + kTileRows * i, tl[i]);
            if (t1 > 0) {
                quantise_trailing();
#pragma unroll
                for (int i = 0; i < D; ++i)
                    if (i < ntl && !in_cache(it.row0 + kTileRows * i)) load_tile(it.row0 + kTileRows * i, tl[i]);
            }
        }

        // the query quantised with quantize_row_i8 in f32 (amax over the 4
        // lanes of qi)
        v4i qa[2];
        double qsc;
        {
            float x[2][16];
            float amax = 0.0f;
#pragma unroll
            for (int sp = 0; sp < 2; ++sp)
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) {
                    const float4 v = qv[sp][t4];
                    x[sp][4 * t4 + 0] = v.x;
                    x[sp][4 * t4 + 1] = v.y;
                    x[sp][4 * t4 + 2] = v.z;
                    x[sp][4 * t4 + 3] = v.w;
                    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
                }
            amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
            amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
            const float qs = amax > 0.0f ? __fdiv_rn(amax, 127.0f) : 1.0f;
            const float iq = __fdiv_rn(1.0f, qs);
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                v4i pk = {0, 0, 0, 0};
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const int c = (int)fminf(fmaxf(rint_div(x[sp][t], qs, iq), -127.0f), 127.0f);
                    pk[t >> 2] |= (c & 0xff) << (8 * (t & 3));
                }
                qa[sp] = pk;
            }
            qsc = (double)qs * kQScale64;
        }
        const int rl = a.ring_len[j], old = a.ring_oldest[j];
        const int evict = max(0, rl + di + 1 - KVQ_RING_WINDOW);
        const int live = kShared ? a.sring[di] : 0;                               // ring slots live before the step
        const int wslot = kShared ? a.swrow[di] - pre - KVQ_RING_WINDOW * di : 0;   // the slot it overwrites
        // every condition evaluated and combined with & and | (no branches:
        // the rows of a lane differ in which case applies)
        auto visible = [&](int p) {
            const int q = p - pre;
            if constexpr (kShared) {
                const int slot = q & (KVQ_RING_WINDOW - 1);
                const bool ring = (q >= 0) & (p < L) & ((q >> 7) == di) & (slot < live) & (slot != wslot);
                return (q < 0) | ring | ((p >= L) & (p - L == di));
            } else {
                const bool ring = (q >= 0) & (p < L) & (((q - old + KVQ_RING_WINDOW) & (KVQ_RING_WINDOW - 1)) >= evict);
                return (q < 0) | ring | ((p >= L) & (p - L <= di));
            }
        };

        float m = -INFINITY, l = 0.0f;
        v4f acc[8];
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) acc[cb] = v4f{0.f, 0.f, 0.f, 0.f};
        // Tile t's arithmetic; with kReload, the whole tile of row rn is then
        // loaded into t: its K side once the scores have read t's, its V side
        // after the value MFMAs (against loading it after the whole tile, on
        // MI355X, 32k R-SWA reference, 8 drafts: 26.5 -> 26.3 us per call).
        auto compute_tile = [&](int r0, Tile& t, int rn, auto reload) {
            constexpr bool kReload = decltype(reload)::value;
            v4i d = {0, 0, 0, 0};
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                const v4i kc = {(int)t.kc[sp].x, (int)t.kc[sp].y, (int)t.kc[sp].z, (int)t.kc[sp].w};
                d = __builtin_amdgcn_mfma_i32_16x16x64_i8(kc, qa[sp], d, 0, 0, 0);
            }
            double s64[4];
            float tmax = -INFINITY;
            bool vis[4];
            if (r0 + kTileRows <= min(pre, it.row1)) {      // reference rows only: every query sees them
#pragma unroll
                for (int r = 0; r < 4; ++r) vis[r] = qvalid;
            } else if (kShared && r0 >= pre && r0 + kTileRows <= min(L, it.row1) &&
                       ((r0 - pre) >> 7) == ((r0 + kTileRows - 1 - pre) >> 7)) {
                // a whole tile of stream ts's ring (wave-uniform): only that
                // stream's queries see it, each of its live slots but the one
                // this step overwrites.  (With the general test below, the
                // waves holding the rings took a third more time per tile: on
                // MI355X, 32k reference and 16 streams, they ended 4-5 us after
                // the others; this path took the call from 33.6 to 29.4 us.)
                const int ts = (r0 - pre) >> 7;
                const int s0 = ((r0 - pre) & (KVQ_RING_WINDOW - 1)) + 4 * kb;
                const bool mine = qvalid & (di == ts);
#pragma unroll
                for (int r = 0; r < 4; ++r) vis[r] = mine & (s0 + r < live) & (s0 + r != wslot);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int p = r0 + 4 * kb + r;
                    vis[r] = qvalid & (p < it.row1) & visible(p);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s64[r] = (double)d[r] * (qsc * (double)t.ks[r]);
                if (vis[r]) tmax = fmaxf(tmax, (float)s64[r]);
            }
            if constexpr (kReload) load_whole_k(rn, t);
            tmax = max_rows(tmax);
            // lazy max: weights stay <= 2^kLazy
            float alpha = 1.0f;
            if (tmax > m + kLazy) {
                alpha = fast_exp2(m - tmax);                 // 0 while m is -inf
                m = tmax;
            }
            if (__any(alpha != 1.0f)) {
                l *= alpha;
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) acc[cb] *= alpha;
            }
            // weights times the rows' V scales (exactly 0 for a row this
            // query does not see, whatever that row's scale holds), in three
            // bf16 parts: B1 = (hi, mid), B2 = (lo, 0)
            uint32_t hi[4], mid[4], lo[4];
            float psum = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float pw = vis[r] ? fast_exp2((float)(s64[r] - (double)m)) : 0.0f;
                psum += pw;
                bf16_split3(vis[r] ? pw * t.vs[r] : 0.0f, hi[r], mid[r], lo[r]);
            }
            l += psum;
            const v4u b1u = {hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), mid[0] | (mid[1] << 16),
                             mid[2] | (mid[3] << 16)};
            const v4u b2u = {lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), 0u, 0u};
            const v8bf b1 = __builtin_bit_cast(v8bf, b1u), b2 = __builtin_bit_cast(v8bf, b2u);
            float vv[4][8];
#pragma unroll
            for (int r = 0; r < 4; ++r) unpack(t.vc[r], vv[r]);
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
                const uint32_t a01 = bf16_pack(vv[0][cb], vv[1][cb]), a23 = bf16_pack(vv[2][cb], vv[3][cb]);
                const v4u au = {a01, a23, a01, a23};
                const v8bf av = __builtin_bit_cast(v8bf, au);
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b1, acc[cb], 0, 0, 0);
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b2, acc[cb], 0, 0, 0);
            }
            if constexpr (kReload) load_whole_v(rn, t);
        };
        // D tiles in flight: slot i holds tile k + i.  The main loop runs full
        // rounds (every slot refilled) while the tiles it loads are whole
        // tiles of cache rows: one straight path whose loop exits only at its
        // head, so that it waits for exactly the loads it uses.  The last
        // tiles (partial, or reading trailing rows) take the general path.
        int k = 0;
        while (k + 2 * D <= nwhole) {
#pragma unroll
            for (int i = 0; i < D; ++i) {
                compute_tile(it.row0 + kTileRows * (k + i), tl[i], it.row0 + kTileRows * (k + D + i), std::true_type{});
            }
            k += D;
        }
        while (k < ntl) {
#pragma unroll
            for (int i = 0; i < D; ++i)
                if (k + i < ntl) {
                    compute_tile(it.row0 + kTileRows * (k + i), tl[i], 0, std::false_type{});
                    if (k + D + i < ntl) load_any(it.row0 + kTileRows * (k + D + i), tl[i]);
                }
            k += D;
        }
        // the piece's partial for each valid query: lane (qi, kb) holds
        // channels 8 (4 kb + r) + cb
        const float lt = sum_rows(l);
        if (qvalid) {
            const size_t ix = (size_t)it.slot * a.nq + qi;
            if (kb == 0) {
                a.ws_ml[ix * 2] = m;
                a.ws_ml[ix * 2 + 1] = lt;
            }
            float* dst = a.ws_acc + ix * kHD + 32 * kb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                *(float4*)(dst + 8 * r) = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
                *(float4*)(dst + 8 * r + 4) = make_float4(acc[4][r], acc[5][r], acc[6][r], acc[7][r]);
            }
        }
    });
}

// Combine of the verify: block (draft i x Q head h x channel chunk, sequence).
__global__ __launch_bounds__(kCombineThreads) void k_combine_verify(const VerifyArgs a) {
    const int chunks = (int)gridDim.x / (a.n_draft * a.n_q_heads);
    const int x = blockIdx.x / chunks, ck = blockIdx.x - x * chunks;
    const int lpg = 32 / chunks, ch0 = 4 * lpg * ck;
    const int j = blockIdx.y, tid = threadIdx.x;
    const int i = x / a.n_q_heads, h = x - i * a.n_q_heads;
    const int b = a.shared ? 0 : a.seq0 + j;              // shared decode: out is [streams][n_q_heads][128]
    const int g = h / a.hpk, hh = h - g * a.hpk;
    const int gl = arg_byte(a.live_slot, g);
    float* o = a.out + (((size_t)b * a.n_draft + i) * a.n_q_heads + h) * kHD + ch0;
    const int nt = a.ntile[j];
    if (gl < 0 || nt == 0) {
        if (tid < lpg) *(float4*)(o + 4 * tid) = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }
    const int sb = a.tile_base[j] + gl * nt;
    const int first = tile_owner(sb, a.n_tiles, a.n_shares);
    const int nch = tile_owner(sb + nt - 1, a.n_tiles, a.n_shares) - first + 1;
    const size_t it0 = (size_t)first + (size_t)j * a.n_live + gl;
    const int vq = i * a.hpk + hh;
    float4 rr;
    if (combine_partials(a.ws_ml + (it0 * a.nq + vq) * 2, a.ws_acc + (it0 * a.nq + vq) * kHD, (size_t)a.nq * 2,
                         (size_t)a.nq * kHD, nch, -INFINITY, lpg, ch0, &rr))
        *(float4*)(o + 4 * tid) = rr;
}

// Threads per combine block: enough sub-groups of lpg lanes that each folds
// at most one batch of partials, at most 512 threads, in whole waves.
int combine_threads(const DecodeArgs& a, int lpg) {
    int nmax = 1;
    for (int j = 0; j < a.n_seq; ++j) {
        const int nt = a.ntile[j];
        if (nt == 0) continue;
        for (int gl = 0; gl < a.n_live; ++gl) {
            const int sb = a.tile_base[j] + gl * nt;
            const int cnt = tile_owner(sb + nt - 1, a.n_tiles, a.n_shares) - tile_owner(sb, a.n_tiles, a.n_shares) + 1;
            nmax = cnt > nmax ? cnt : nmax;
        }
    }
    int groups = (nmax + kCombineBatch - 1) / kCombineBatch;
    const int gmax = kCombineThreads / lpg;
    groups = groups < 1 ? 1 : (groups > gmax ? gmax : groups);
    return (lpg * groups + 63) / 64 * 64;          // whole waves
}

// Waves of a decode kernel that are resident on the current device at once
// (compute units x workgroups per unit x 4), at most kMaxWaves; cached per
// device and kernel.  0 on a runtime error.
constexpr int kMaxDevices = 64;
int resident_waves(const void* kernel, int which) {
    // host threads may race to fill an entry; they all store the same value
    static std::atomic<int> cache[kMaxDevices][52];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    std::atomic<int>& c = cache[dev][which];
    int v = c.load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kWaves * 64, 0) != hipSuccess) return 0;
        const int64_t wv = (int64_t)cus * per_cu * kWaves;
        v = (int)(wv < 1 ? 1 : (wv > kMaxWaves ? kMaxWaves : wv));
        c.store(v, std::memory_order_relaxed);
    }
    return v;
}

// SIMDs of the current device (compute units x 4), at most kMaxWaves (the
// share bound the workspace is sized for); cached per device; 0 on a runtime
// error.
int simd_count() {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        v = cus < 1 ? 1 : (cus * 4 > kMaxWaves ? kMaxWaves : cus * 4);
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

int hpk_index(int hpk) { return hpk == 1 ? 0 : hpk == 2 ? 1 : hpk == 4 ? 2 : 3; }

// Shares rounded down to a multiple of the segment count when every
// (sequence, live head) segment has the same number of tiles (one sequence,
// or a batch of equal lengths): the split then puts every share inside one
// segment, and no wave pays a second piece's set-up, drain and partial.
// Used by the query-batched kernels and the q8 / int8 decode, whose piece
// set-up (query quantisation, first tiles' latency) is long: on MI355X, in
// the 32k R-SWA int8 verify the 8 waves whose shares crossed a head boundary
// ended 10 us after the others, and aligned shares took the call from 35.5
// to 30.8 us (shared decode 43.4 to 38.9 us).  The f32 decode got slower with
// it (R-SWA step 57.1 against 65.4 us: the shares become unequal by a tile).
template <class Args>
int align_shares(const Args& a, int shares) {
    int nt = -1;
    for (int j = 0; j < a.n_seq; ++j) {
        if (a.ntile[j] == 0) continue;
        if (nt >= 0 && a.ntile[j] != nt) return shares;
        nt = a.ntile[j];
    }
    int nseg = 0;
    for (int j = 0; j < a.n_seq; ++j) nseg += a.ntile[j] > 0 ? a.n_live : 0;
    if (nseg == 0 || nseg > shares) return shares;
    return shares / nseg * nseg;
}

// Cache kinds of the decode launcher.
constexpr int kF32 = 0, kQ8k = 1, kI8k = 2;

// The kernel instance for a group size, cache kind, soft-cap switch and
// value pass (mf: on the matrix cores; groups of 1 or 2 heads have only the
// VALU one).
template <int HPK, bool kCap, bool kI8>
const void* q8_kernel(bool mf) {
    if constexpr (HPK >= 4)
        return mf ? (const void*)k_decode_q8<HPK, kCap, kI8, true> : (const void*)k_decode_q8<HPK, kCap, kI8, false>;
    return (const void*)k_decode_q8<HPK, kCap, kI8, false>;
}
template <int HPK, int kKind>
const void* decode_kernel(bool cap, bool mf) {
    if (kKind == kI8k) return q8_kernel<HPK, false, true>(mf);
    if (kKind == kQ8k) return cap ? q8_kernel<HPK, true, false>(mf) : q8_kernel<HPK, false, false>(mf);
    return cap ? (const void*)k_decode_f32<HPK, true> : (const void*)k_decode_f32<HPK, false>;
}

// Shares per launch: one per resident wave for the q8 kernel (a wave keeps
// one 4.4-KB tile in flight beside the one it computes) -- but one per SIMD
// when that would leave fewer than kQ8MinTilesPerWave tiles per resident
// wave: a short launch is then dominated by each share's query set-up and
// partial (measured on MI355X, one 8192-row sequence, 32 Q / 8 KV heads,
// 4096 tiles: one share per resident wave, 3072 shares, 21.2 us; 2048 shares
// 18.2 us; 1024, one per SIMD, 16.4 us; 1365 or 682 shares, not a whole
// number of workgroups per compute unit, 21.2 and 21.6 us) -- and one per SIMD for the
// f32 kernel: a wave's 16-KB tiles keep HBM busy with one wave per SIMD, and
// fewer shares make the combine cheaper (measured on MI355X, 4 x 10 heads x
// 32k rows, the R-SWA step: one share per 2 SIMDs 89.0 us, per SIMD 57.9 us,
// 2 per SIMD 59.0 us; the combine alone 5.0 us at one per SIMD and 9.1 us at
// 4 per SIMD) -- except a short f32 launch (fewer than two tiles per SIMD),
// which takes one tile per wave: with one wave per SIMD its waves spend the
// kernel in the dependent shuffles of their tiles, and more waves overlap them.

// (Also measured on the R-SWA step on the int8 mirror, 5 tiles per resident
// wave: one share per SIMD 23.7 against 22.3 us; two per SIMD 22.3 us, and
// two per SIMD on the short q8 launch above 16.6 against 15.1 us.)
constexpr int kQ8MinTilesPerWave = 4;
// The q8 / int8 value pass goes to the matrix cores only when a launch has
// at least this many tiles per resident wave; below that the VALU instance
// runs.  Measured on MI355X, 32 Q / 8 KV heads, q8 (matrix cores against
// VALU): one 8192-row sequence 15.8 / 14.8 us, one of 131072 rows (11 tiles
// per wave) 60.0 / 58.6, 4 x 32768 rows (21 per wave) 59.5 / 57.7, 8 x 32768
// (43 per wave) 100.1 / 100.1, the 64-sequence batch of 1024..32768 rows
// (167 per wave) 363.7 / 366.3; int8 alike.
#ifndef KVQ_Q8_PV_MIN_TILES
#define KVQ_Q8_PV_MIN_TILES 48
#endif

template <int kKind>
hipError_t launch_decode(const DecodeArgs& args, hipStream_t s) {
    constexpr bool kQ8 = kKind != kF32;
    DecodeArgs a = args;
    a.n_shares = 1;
    if (a.n_tiles > 0) {
        const bool cap = a.softcap2 > 0.0;
        const void* fn = nullptr;
        auto pick = [&](bool mf) -> const void* {
            switch (a.hpk) {
                case 1: return decode_kernel<1, kKind>(cap, mf);
                case 2: return decode_kernel<2, kKind>(cap, mf);
                case 4: return decode_kernel<4, kKind>(cap, mf);
                case 8: return decode_kernel<8, kKind>(cap, mf);
                default: return nullptr;
            }
        };
        const int which = 8 * kKind + 4 * cap + hpk_index(a.hpk);
        fn = pick(true);
        if (fn == nullptr) return hipErrorInvalidValue;
        int shares = kQ8 ? resident_waves(fn, which) : simd_count();
        if (kQ8 && a.hpk >= 4 && shares > 0 && (int64_t)a.n_tiles < (int64_t)KVQ_Q8_PV_MIN_TILES * shares) {
            fn = pick(false);
            shares = resident_waves(fn, which + 28);   // entries 28.. (24..27: verify)
        }
        if (kQ8 && shares > 0 && a.n_tiles < kQ8MinTilesPerWave * shares) shares = simd_count();
        // f32, short launch: one tile per wave (gqa 4096 rows x 6 heads: 16.8 -> 15.2 us per call)
        if (!kQ8 && shares > 0 && a.n_tiles < 2 * shares) shares = a.n_tiles;
        if (shares == 0) return hipErrorInvalidDevice;
        if (kQ8) shares = align_shares(a, shares);
        a.n_shares = shares < a.n_tiles ? shares : a.n_tiles;
        const dim3 grid((a.n_shares + kWaves - 1) / kWaves), block(kWaves * 64);
        void* kargs[] = {&a};
        const hipError_t e = hipLaunchKernel(fn, grid, block, kargs, 0, s);
        if (e != hipSuccess) return e;
    }
    // the i8 kind has no column field to apply
    const int chunks = combine_chunks(a.n_q_heads * a.n_seq);
    hipLaunchKernelGGL(k_combine<kKind == kQ8k>, dim3(a.n_q_heads * chunks, a.n_seq),
                       dim3(combine_threads(a, 32 / chunks)), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s) { return launch_decode<kF32>(a, s); }
hipError_t launch_decode_i8(const DecodeArgs& a, hipStream_t s) { return launch_decode<kI8k>(a, s); }

namespace {

// The query-batched launch: the kernel, then its combine.  which: the
// resident-wave cache entry of the kernel; one share per wps resident waves,
// or one per SIMD when wps is 0; align: shares aligned to equal segments.
hipError_t launch_query_batched(const VerifyArgs& args, const void* fn, int which, int wps, bool align,
                                hipStream_t s) {
    VerifyArgs a = args;
    a.n_shares = 1;
    if (a.n_tiles > 0) {                          // zero only when every group is dead
        const int wv = wps ? resident_waves(fn, which) : simd_count();
        if (wv == 0) return hipErrorInvalidDevice;
        const int shares0 = wps ? (wv + wps - 1) / wps : wv;
        const int shares = align ? align_shares(a, shares0) : shares0;
        a.n_shares = shares < a.n_tiles ? shares : a.n_tiles;
        const dim3 grid((a.n_shares + kWaves - 1) / kWaves), block(kWaves * 64);
        void* kargs[] = {&a};
        const hipError_t e = hipLaunchKernel(fn, grid, block, kargs, 0, s);
        if (e != hipSuccess) return e;
    }
    int nmax = 1;
    for (int j = 0; j < a.n_seq; ++j)
        for (int gl = 0; gl < a.n_live; ++gl) {
            const int sb = a.tile_base[j] + gl * a.ntile[j];
            const int cnt = tile_owner(sb + a.ntile[j] - 1, a.n_tiles, a.n_shares) -
                            tile_owner(sb, a.n_tiles, a.n_shares) + 1;
            nmax = cnt > nmax ? cnt : nmax;
        }
    const int chunks = combine_chunks(a.n_draft * a.n_q_heads * a.n_seq);
    const int lpg = 32 / chunks;
    int groups = (nmax + kCombineBatch - 1) / kCombineBatch;
    const int gmax = kCombineThreads / lpg;
    groups = groups < 1 ? 1 : (groups > gmax ? gmax : groups);
    hipLaunchKernelGGL(k_combine_verify, dim3(a.n_draft * a.n_q_heads * chunks, a.n_seq), dim3((lpg * groups + 63) / 64 * 64), 0, s,
                       a);
    return hipGetLastError();
}

}  // namespace

// Shares: up to 16 queries per row make these waves compute-heavy, unlike the
// single-query decode.  Measured on MI355X (32k R-SWA reference): the f32
// kernel at 2 waves/SIMD was fastest with one share per 2 resident waves,
// i.e. one per SIMD (verify 70.0 -> 68.0 us), which the verify now takes
// directly at one wave per SIMD.  The i8 kernel runs one share per SIMD with
// KVQ_VI8_DEPTH tiles in flight and shares aligned to the heads: verify 30.8
// us, shared decode 38.9 us (one share per resident wave, 3 waves/SIMD and
// one tile in flight: 35.5 and 43.4 us).
// Adds pad tiles, which hold no rows, to the end of every segment of a.
bool pad_segments(VerifyArgs& a, int pad) {
    if (pad <= 0) return true;
    int64_t tiles = 0;
    for (int j = 0; j < a.n_seq; ++j) {
        a.tile_base[j] = (int32_t)tiles;
        if (a.ntile[j] > 0) a.ntile[j] += pad;
        tiles += (int64_t)a.ntile[j] * a.n_live;
    }
    if (tiles >= ((int64_t)1 << 31)) return false;
    a.tile_base[a.n_seq] = (int32_t)tiles;
    a.n_tiles = (int)tiles;
    return true;
}

// The f32 kernel, likewise (shares aligned to the heads, padding tiles per
// segment; measured on MI355X, 32k R-SWA reference: verify 67.3 -> 65.4 us,
// shared decode 72.4 -> 70.7 us).
#ifndef KVQ_VF32_PAD
#define KVQ_VF32_PAD 8
#endif
#ifndef KVQ_VF32S_PAD
#define KVQ_VF32S_PAD 16
#endif
#ifndef KVQ_VF32_ALIGN
#define KVQ_VF32_ALIGN 1
#endif
hipError_t launch_verify_f32(const VerifyArgs& args, hipStream_t s) {
    VerifyArgs a = args;
    if (!pad_segments(a, a.shared ? KVQ_VF32S_PAD : KVQ_VF32_PAD)) return hipErrorInvalidValue;
    // the shared decode: one share per 2 resident waves; the verify: one per SIMD
    return a.shared ? launch_query_batched(a, reinterpret_cast<const void*>(k_verify_f32<true>), 25, 2, KVQ_VF32_ALIGN, s)
                    : launch_query_batched(a, reinterpret_cast<const void*>(k_verify_f32<false>), 24, 0, KVQ_VF32_ALIGN, s);
}

#ifndef KVQ_VI8_WPS
#define KVQ_VI8_WPS 0
#endif
#ifndef KVQ_VI8S_WPS
#define KVQ_VI8S_WPS 0
#endif
// Padding tiles per segment: the wave whose share holds a segment's last
// tiles also quantises its trailing rows (and, in the shared decode, reads
// the rings, whose visibility costs more per tile); padding tiles at the end
// of every segment, which hold no rows, give that share fewer real tiles.
// Measured on MI355X (32k R-SWA reference, 10 heads): that wave ended 5 us
// (verify) and 11 us (shared decode) after the median one; with padding
// (verify, shared) 0/0 tiles 30.4 / 39.0 us per call, 4/6 28.0 / 35.2,
// 8/14 26.3 / 33.5, 10/18 26.2 / 33.6.
#ifndef KVQ_VI8_PAD
#define KVQ_VI8_PAD 9
#endif
#ifndef KVQ_VI8S_PAD
#define KVQ_VI8S_PAD 14
#endif
hipError_t launch_verify_i8(const VerifyArgs& args, hipStream_t s) {
    VerifyArgs a = args;
    if (!pad_segments(a, a.shared ? KVQ_VI8S_PAD : KVQ_VI8_PAD)) return hipErrorInvalidValue;
    return a.shared ? launch_query_batched(a, reinterpret_cast<const void*>(k_verify_i8<true>), 27, KVQ_VI8S_WPS, true, s)
                    : launch_query_batched(a, reinterpret_cast<const void*>(k_verify_i8<false>), 26, KVQ_VI8_WPS, true, s);
}

hipError_t launch_decode_q8(const DecodeArgs& a, hipStream_t s) { return launch_decode<kQ8k>(a, s); }

}  // namespace kvq
