// kvq_decode.hip -- split-K single-query decode attention for gfx950.
//
// One workgroup (256 threads = 4 wave64s) per work item = one chunk of rows
// of one (sequence, live KV head).  Every K and V row of the chunk is read
// from HBM exactly once and serves all hpk Q heads of the GQA group
// (cortiq-engine 0.3.4 kv_cache.rs, LayerKvCache::attend_group: each stored
// row read once for all heads of its group).  Each wave streams 16-byte
// loads, keeps an online-softmax state per Q head in registers (franken_ocr
// 0.8.0 rswa.rs, fold: rescale the running sum and accumulator when the
// running max grows, never materialising the score row), the four waves
// merge in LDS, and the item writes one partial (max, sum, acc[128]) per Q
// head.  A second kernel merges the partials of a (sequence, Q head) with
// the same rescaling and divides.
//
// Scores are kept in log2 units (the query is pre-scaled by
// log2(e)/sqrt(128)) so every exponential is one v_exp_f32.
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kQScale = 0.12751743082459868f;   // log2(e) / sqrt(128)
constexpr double kQScale64 = 0.12751743082459868;
constexpr int kWaves = 4;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// Sequence slot of a work item: the last j with item_base[j] <= item.
__device__ __forceinline__ int find_seq(const DecodeArgs& a, int item) {
    int lo = 0, hi = a.n_seq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.item_base[mid] <= item) lo = mid; else hi = mid - 1;
    }
    return lo;
}

struct Item {
    int j, b, gl, g, row0, row1;
    size_t hrow;     // first storage row of the (sequence, live head)
};

__device__ __forceinline__ Item decode_item(const DecodeArgs& a) {
    Item it;
    const int item = blockIdx.x;
    it.j = find_seq(a, item);
    const int nch = a.nchunk[it.j];
    const int rem = item - a.item_base[it.j];
    it.gl = rem / nch;
    const int ch = rem - it.gl * nch;
    it.b = a.seq0 + it.j;
    it.g = a.live_head[it.gl];
    it.row0 = ch * a.chunk;
    it.row1 = min(it.row0 + a.chunk, a.len[it.j]);
    it.hrow = ((size_t)it.b * a.n_live + it.gl) * a.capacity;
    return it;
}

// Merge the four waves' states in LDS and write the item's partials.
template <int HPK>
__device__ __forceinline__ void write_partials(const DecodeArgs& a, float (*sm_acc)[HPK][kHD],
                                               float (*sm_ml)[HPK][2]) {
    __syncthreads();
    const int item = blockIdx.x;
    for (int t = threadIdx.x; t < HPK * kHD; t += kWaves * 64) {
        const int h = t / kHD, d = t - h * kHD;
        float M = sm_ml[0][h][0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_ml[w][h][0]);
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float e = fast_exp2(sm_ml[w][h][0] - M);
            L += e * sm_ml[w][h][1];
            A += e * sm_acc[w][h][d];
        }
        const size_t ix = (size_t)item * HPK + h;
        a.ws_acc[ix * kHD + d] = A;
        if (d == 0) {
            a.ws_ml[ix * 2] = M;
            a.ws_ml[ix * 2 + 1] = L;
        }
    }
}

// ---------------------------------------------------------------------------
// f32 cache.  Lane layout: half = lane >> 5 picks the row of a pair, seg =
// lane & 31 the 4 channels [4 seg, 4 seg + 4).  One 16-byte load per lane
// covers two consecutive 512-byte rows; a wave takes 16 rows per step.
// ---------------------------------------------------------------------------
// Sum 8 per-lane partials over the 32 lanes of a half so that lanes with
// (seg >> 2) == i end with the total of partial i (transpose-reduce: 9
// exchanges instead of 40).
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

template <int HPK>
__global__ __launch_bounds__(256) void k_decode_f32(const DecodeArgs a) {
    __shared__ float sm_acc[kWaves][HPK][kHD];
    __shared__ float sm_ml[kWaves][HPK][2];
    const Item it = decode_item(a);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int half = lane >> 5, seg = lane & 31;
    const float* K = a.k + it.hrow * kHD;
    const float* V = a.v + it.hrow * kHD;
    const int wrow = a.wrow[it.j];
    const bool has_w = wrow >= it.row0 && wrow < it.row1;
    const float* kn = has_w ? a.k_new + ((size_t)it.b * a.n_kv_heads + it.g) * kHD : K;
    const float* vn = has_w ? a.v_new + ((size_t)it.b * a.n_kv_heads + it.g) * kHD : V;

    // R-SWA ring write: this item owns the row, nobody else reads it.
    if (has_w && tid < 32) {
        *(float4*)(a.k_store + (it.hrow + wrow) * kHD + 4 * tid) = *(const float4*)(kn + 4 * tid);
        *(float4*)(a.v_store + (it.hrow + wrow) * kHD + 4 * tid) = *(const float4*)(vn + 4 * tid);
    }

    float4 qv[HPK];
#pragma unroll
    for (int h = 0; h < HPK; ++h) {
        const float4 t = *(const float4*)(a.q + ((size_t)it.b * a.n_q_heads + it.g * HPK + h) * kHD + 4 * seg);
        qv[h] = make_float4(t.x * kQScale, t.y * kQScale, t.z * kQScale, t.w * kQScale);
    }
    float m[HPK], l[HPK];
    float4 acc[HPK];
#pragma unroll
    for (int h = 0; h < HPK; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
        acc[h] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    for (int r = it.row0 + wave * 16; r < it.row1; r += kWaves * 16) {
        float4 kx[8], vx[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = min(r + 2 * i + half, it.row1 - 1);
            const bool w = has_w && row == wrow;
            kx[i] = *(const float4*)((w ? kn : K + (size_t)row * kHD) + 4 * seg);
            vx[i] = *(const float4*)((w ? vn : V + (size_t)row * kHD) + 4 * seg);
        }
        const int myrow = r + 2 * (seg >> 2) + half;
#pragma unroll
        for (int h = 0; h < HPK; ++h) {
            float part[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float d = qv[h].x * kx[i].x;
                d = fmaf(qv[h].y, kx[i].y, d);
                d = fmaf(qv[h].z, kx[i].z, d);
                d = fmaf(qv[h].w, kx[i].w, d);
                part[i] = d;
            }
            float s = reduce8_over32(part, seg);
            if (myrow >= it.row1) s = -INFINITY;
            const float mnew = fmaxf(m[h], wave_max(s));
            const float alpha = fast_exp2(m[h] - mnew);
            const float p = fast_exp2(s - mnew);
            l[h] = l[h] * alpha + ((seg & 3) == 0 ? p : 0.0f);
            float4 ac = make_float4(acc[h].x * alpha, acc[h].y * alpha, acc[h].z * alpha, acc[h].w * alpha);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float pi = __shfl(p, half * 32 + 4 * i, 64);
                ac.x = fmaf(pi, vx[i].x, ac.x);
                ac.y = fmaf(pi, vx[i].y, ac.y);
                ac.z = fmaf(pi, vx[i].z, ac.z);
                ac.w = fmaf(pi, vx[i].w, ac.w);
            }
            acc[h] = ac;
            m[h] = mnew;
        }
    }

#pragma unroll
    for (int h = 0; h < HPK; ++h) {
        const float lt = wave_sum(l[h]);
        float4 at = acc[h];
        at.x += __shfl_xor(at.x, 32, 64);
        at.y += __shfl_xor(at.y, 32, 64);
        at.z += __shfl_xor(at.z, 32, 64);
        at.w += __shfl_xor(at.w, 32, 64);
        if (half == 0) *(float4*)&sm_acc[wave][h][4 * seg] = at;
        if (lane == 0) {
            sm_ml[wave][h][0] = m[h];
            sm_ml[wave][h][1] = lt;
        }
    }
    write_partials<HPK>(a, sm_acc, sm_ml);
}

// ---------------------------------------------------------------------------
// q8 cache.  Lane layout: ri = lane >> 3 picks one of 8 rows, seg = lane & 7
// the 16 channels [16 seg, 16 seg + 16) (half of a 32-channel K group).  One
// 16-byte load per lane covers eight consecutive 128-byte int8 rows; a wave
// takes 32 rows per step.
//
// Scores are computed exactly.  The query side of a score, q (.) kcol
// ([P1] attend: score = s_k * <q (.) col_k, k_q>), is split once per work
// item into four balanced base-128 int8 digits relative to a power of two
// per (Q head, K group): qc = 2^(e-27) * (((d0*128 + d1)*128 + d2)*128 + d3)
// with |qc - that| <= 2^(e-28).  Each digit's dot with the int8 codes is an
// exact i32 (v_dot4), the digits combine exactly in f64, and the K group
// scale and 1/sqrt(128) multiply in f64; the score stays f64 until the
// running max is subtracted.  V codes become f32 with one sign-extending byte
// convert each, V row scales fold into the softmax weight, and the V column
// field is applied once in the combine ([P1] attend: acc (.) vcol at the end).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void unpack16(const uint4 x, float (&f)[16]) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f[4 * k + 0] = (float)(int8_t)(w[k] & 0xffu);
        f[4 * k + 1] = (float)(int8_t)((w[k] >> 8) & 0xffu);
        f[4 * k + 2] = (float)(int8_t)((w[k] >> 16) & 0xffu);
        f[4 * k + 3] = (float)((int32_t)w[k] >> 24);
    }
}

__device__ __forceinline__ double shfl_xor_f64(double x, int m) {
    const int2 v = *reinterpret_cast<int2*>(&x);
    int2 r;
    r.x = __shfl_xor(v.x, m, 64);
    r.y = __shfl_xor(v.y, m, 64);
    return *reinterpret_cast<double*>(&r);
}

// Sum 4 per-lane partials over the 8 lanes of a row group so that lanes with
// (seg >> 1) == i end with the total of partial i.
__device__ __forceinline__ double reduce4_over8_f64(const double (&v)[4], int seg) {
    const bool b2 = seg & 4, b1 = seg & 2;
    double x[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const double keep = b2 ? v[i + 2] : v[i];
        const double send = b2 ? v[i] : v[i + 2];
        x[i] = keep + shfl_xor_f64(send, 4);
    }
    double z = (b1 ? x[1] : x[0]) + shfl_xor_f64(b1 ? x[0] : x[1], 2);
    z += shfl_xor_f64(z, 1);
    return z;
}

// One balanced base-128 digit: x = 128 * next + digit, digit in [-64, 63].
__device__ __forceinline__ int take_digit(int& x) {
    const int d = ((x + 64) & 127) - 64;
    x = (x - d) >> 7;
    return d;
}

template <int HPK>
__global__ __launch_bounds__(256) void k_decode_q8(const DecodeArgs a) {
    __shared__ float sm_acc[kWaves][HPK][kHD];
    __shared__ float sm_ml[kWaves][HPK][2];
    const Item it = decode_item(a);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ri = lane >> 3, seg = lane & 7, grp = seg >> 1;
    const int8_t* KQ = a.kq + it.hrow * kHD;
    const float* KS = a.ks + it.hrow * kKScales;
    const int8_t* VQ = a.vq + it.hrow * kHD;
    const float* VS = a.vs + it.hrow;
    const bool frz = a.frozen[it.j] != 0;
    const float* kcol = a.kcol + ((size_t)it.b * a.n_live + it.gl) * kHD + 16 * seg;

    // Query digits: dig[h][j][w] packs digit j of channels 16 seg + 4w .. +3.
    int dig[HPK][4][4];
    double gscale[HPK];            // 2^(e-27) * log2(e)/sqrt(128) for this lane's group
#pragma unroll
    for (int h = 0; h < HPK; ++h) {
        const float* qp = a.q + ((size_t)it.b * a.n_q_heads + it.g * HPK + h) * kHD + 16 * seg;
        double qc[16];
        double amax = 0.0;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const float4 t = *(const float4*)(qp + 4 * c4);
            float4 cc = make_float4(1.f, 1.f, 1.f, 1.f);
            if (frz) cc = *(const float4*)(kcol + 4 * c4);
            qc[4 * c4 + 0] = (double)t.x * (double)cc.x;      // exact products
            qc[4 * c4 + 1] = (double)t.y * (double)cc.y;
            qc[4 * c4 + 2] = (double)t.z * (double)cc.z;
            qc[4 * c4 + 3] = (double)t.w * (double)cc.w;
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) amax = fmax(amax, fabs(qc[c]));
        amax = fmax(amax, shfl_xor_f64(amax, 1));             // the other half of the K group
        int e = 0;
        (void)frexp(amax, &e);                                 // amax < 2^e
        const double up = ldexp(1.0, 27 - e);
        gscale[h] = ldexp(kQScale64, e - 27);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            int pk[4] = {0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                int x = (int)rint(qc[4 * w + c] * up);          // |x| <= 2^27
                const int d3 = take_digit(x);
                const int d2 = take_digit(x);
                const int d1 = take_digit(x);
                const int d0 = x;                               // |d0| <= 64
                pk[0] |= (d0 & 0xff) << (8 * c);
                pk[1] |= (d1 & 0xff) << (8 * c);
                pk[2] |= (d2 & 0xff) << (8 * c);
                pk[3] |= (d3 & 0xff) << (8 * c);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) dig[h][j][w] = pk[j];
        }
    }
    float m[HPK], l[HPK], acc[HPK][16];
#pragma unroll
    for (int h = 0; h < HPK; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
#pragma unroll
        for (int c = 0; c < 16; ++c) acc[h][c] = 0.0f;
    }

    for (int r = it.row0 + wave * 32; r < it.row1; r += kWaves * 32) {
        uint4 kx[4], vx[4];
        float ksv[4], vsv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const size_t row = (size_t)min(r + 8 * i + ri, it.row1 - 1);
            kx[i] = *(const uint4*)(KQ + row * kHD + 16 * seg);
            ksv[i] = KS[row * kKScales + grp];
            vx[i] = *(const uint4*)(VQ + row * kHD + 16 * seg);
            vsv[i] = VS[row];
        }
        double part[HPK][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double ks64 = (double)ksv[i];
#pragma unroll
            for (int h = 0; h < HPK; ++h) {
                int sj[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    int t = __builtin_amdgcn_sdot4(dig[h][j][0], (int)kx[i].x, 0, false);
                    t = __builtin_amdgcn_sdot4(dig[h][j][1], (int)kx[i].y, t, false);
                    t = __builtin_amdgcn_sdot4(dig[h][j][2], (int)kx[i].z, t, false);
                    t = __builtin_amdgcn_sdot4(dig[h][j][3], (int)kx[i].w, t, false);
                    sj[j] = t;
                }
                double x = (double)sj[0];
                x = fma(x, 128.0, (double)sj[1]);
                x = fma(x, 128.0, (double)sj[2]);
                x = fma(x, 128.0, (double)sj[3]);
                part[h][i] = x * (ks64 * gscale[h]);
            }
        }
        const int myrow = r + 8 * (seg >> 1) + ri;
        float pw[HPK][4];
#pragma unroll
        for (int h = 0; h < HPK; ++h) {
            double s = reduce4_over8_f64(part[h], seg);
            if (myrow >= it.row1) s = -INFINITY;
            const float mnew = fmaxf(m[h], wave_max((float)s));
            const float alpha = fast_exp2(m[h] - mnew);
            const float p = fast_exp2((float)(s - (double)mnew));
            l[h] = l[h] * alpha + ((seg & 1) == 0 ? p : 0.0f);
#pragma unroll
            for (int c = 0; c < 16; ++c) acc[h][c] *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) pw[h][i] = __shfl(p, ri * 8 + 2 * i, 64) * vsv[i];
            m[h] = mnew;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float vf[16];
            unpack16(vx[i], vf);
#pragma unroll
            for (int h = 0; h < HPK; ++h) {
#pragma unroll
                for (int c = 0; c < 16; ++c) acc[h][c] = fmaf(pw[h][i], vf[c], acc[h][c]);
            }
        }
    }

#pragma unroll
    for (int h = 0; h < HPK; ++h) {
        const float lt = wave_sum(l[h]);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            float x = acc[h][c];
            x += __shfl_xor(x, 8, 64);
            x += __shfl_xor(x, 16, 64);
            x += __shfl_xor(x, 32, 64);
            acc[h][c] = x;
        }
        if (ri == 0) {
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4)
                *(float4*)&sm_acc[wave][h][16 * seg + 4 * c4] =
                    make_float4(acc[h][4 * c4], acc[h][4 * c4 + 1], acc[h][4 * c4 + 2], acc[h][4 * c4 + 3]);
        }
        if (lane == 0) {
            sm_ml[wave][h][0] = m[h];
            sm_ml[wave][h][1] = lt;
        }
    }
    write_partials<HPK>(a, sm_acc, sm_ml);
}

// ---------------------------------------------------------------------------
// Combine: per (sequence, Q head), merge the chunk partials with the same
// rescaling as the fold, divide, and apply the V column field (q8 only).
// Q heads of dead groups, and sequences with no rows, get zeros.
// 256 threads: a block max over the chunk maxima, then 8 sub-groups of 32
// lanes (a float4 of channels each) stride over the chunks, merged in LDS.
// ---------------------------------------------------------------------------
constexpr int kCombineThreads = 256;
constexpr int kCombineGroups = kCombineThreads / 32;

template <bool kQ8>
__global__ __launch_bounds__(kCombineThreads) void k_combine(const DecodeArgs a) {
    __shared__ float sm_red[kCombineThreads / 64];
    __shared__ float4 sm_acc[kCombineGroups][32];
    __shared__ float sm_l[kCombineGroups];
    const int h = blockIdx.x, j = blockIdx.y, tid = threadIdx.x;
    const int b = a.seq0 + j;
    const int g = h / a.hpk, hh = h - g * a.hpk;
    const int gl = a.live_slot[g];
    float* o = a.out + ((size_t)b * a.n_q_heads + h) * kHD;
    if (gl < 0 || a.len[j] == 0) {
        if (tid < 32) *(float4*)(o + 4 * tid) = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }
    const int nch = a.nchunk[j];
    const size_t it0 = (size_t)a.item_base[j] + (size_t)gl * nch;
    const float* ml = a.ws_ml + (it0 * a.hpk + hh) * 2;          // stride hpk*2 per chunk
    const float* acc = a.ws_acc + (it0 * a.hpk + hh) * kHD;      // stride hpk*128 per chunk
    const size_t mstride = (size_t)a.hpk * 2, astride = (size_t)a.hpk * kHD;

    float M = -INFINITY;
    for (int c = tid; c < nch; c += kCombineThreads) M = fmaxf(M, ml[c * mstride]);
    M = wave_max(M);
    if ((tid & 63) == 0) sm_red[tid >> 6] = M;
    __syncthreads();
    M = fmaxf(fmaxf(sm_red[0], sm_red[1]), fmaxf(sm_red[2], sm_red[3]));

    const int sg = tid >> 5, lane = tid & 31;
    float L = 0.0f;
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int c = sg; c < nch; c += kCombineGroups) {
        const float e = fast_exp2(ml[c * mstride] - M);
        const float4 x = *(const float4*)(acc + c * astride + 4 * lane);
        L = fmaf(e, ml[c * mstride + 1], L);
        A.x = fmaf(e, x.x, A.x);
        A.y = fmaf(e, x.y, A.y);
        A.z = fmaf(e, x.z, A.z);
        A.w = fmaf(e, x.w, A.w);
    }
    sm_acc[sg][lane] = A;
    if (lane == 0) sm_l[sg] = L;
    __syncthreads();
    if (tid < 32) {
        float Lt = 0.0f;
        float4 At = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int k = 0; k < kCombineGroups; ++k) {
            Lt += sm_l[k];
            At.x += sm_acc[k][tid].x;
            At.y += sm_acc[k][tid].y;
            At.z += sm_acc[k][tid].z;
            At.w += sm_acc[k][tid].w;
        }
        const float inv = 1.0f / Lt;
        float4 r = make_float4(At.x * inv, At.y * inv, At.z * inv, At.w * inv);
        if (kQ8 && a.frozen[j]) {
            const float4 vc = *(const float4*)(a.vcol + ((size_t)b * a.n_live + gl) * kHD + 4 * tid);
            r.x *= vc.x;
            r.y *= vc.y;
            r.z *= vc.z;
            r.w *= vc.w;
        }
        *(float4*)(o + 4 * tid) = r;
    }
}

}  // namespace

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s) {
    if (a.n_items > 0) {
        const dim3 grid(a.n_items), block(kWaves * 64);
        switch (a.hpk) {
            case 1: hipLaunchKernelGGL(k_decode_f32<1>, grid, block, 0, s, a); break;
            case 2: hipLaunchKernelGGL(k_decode_f32<2>, grid, block, 0, s, a); break;
            case 4: hipLaunchKernelGGL(k_decode_f32<4>, grid, block, 0, s, a); break;
            case 8: hipLaunchKernelGGL(k_decode_f32<8>, grid, block, 0, s, a); break;
            default: return hipErrorInvalidValue;
        }
    }
    hipLaunchKernelGGL(k_combine<false>, dim3(a.n_q_heads, a.n_seq), dim3(kCombineThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode_q8(const DecodeArgs& a, hipStream_t s) {
    if (a.n_items > 0) {
        const dim3 grid(a.n_items), block(kWaves * 64);
        switch (a.hpk) {
            case 1: hipLaunchKernelGGL(k_decode_q8<1>, grid, block, 0, s, a); break;
            case 2: hipLaunchKernelGGL(k_decode_q8<2>, grid, block, 0, s, a); break;
            case 4: hipLaunchKernelGGL(k_decode_q8<4>, grid, block, 0, s, a); break;
            case 8: hipLaunchKernelGGL(k_decode_q8<8>, grid, block, 0, s, a); break;
            default: return hipErrorInvalidValue;
        }
    }
    hipLaunchKernelGGL(k_combine<true>, dim3(a.n_q_heads, a.n_seq), dim3(kCombineThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
