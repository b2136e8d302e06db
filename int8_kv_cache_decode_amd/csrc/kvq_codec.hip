// kvq_codec.hip -- row append (f32 copy, q8_2f quantise) and the q8_2f
// column-field freeze with requantisation, for gfx950.
//
// The q8_2f codec has exactly one correct output per input, fixed by the
// f32 steps of cortiq-engine 0.3.4 kv_cache.rs (LayerKvCache::quant_row and
// LayerKvCache::freeze_cols).  Every operation here is one IEEE single
// rounding: correctly-rounded division (__fdiv_rn) and square root (sqrtf),
// round half away from zero (roundf, the page's f32::round), and no fused
// multiply-add (contraction is off for this whole file; it is also built
// with -ffp-contract=off).
#pragma clang fp contract(off)

#include <algorithm>

#include "kvq_internal.h"

namespace kvq {
namespace {

// One quantised code: clamp(round_half_away(r / s), -127, 127).
__device__ __forceinline__ int8_t quant_code(float r, float s) {
    float c = roundf(__fdiv_rn(r, s));
    c = fminf(fmaxf(c, -127.0f), 127.0f);
    return (int8_t)(int)c;
}

// s = max(absmax / 127, 1e-12).
__device__ __forceinline__ float group_scale(float absmax) {
    return fmaxf(__fdiv_rn(absmax, 127.0f), 1e-12f);
}

// Max over aligned groups of `width` lanes (width a power of two <= 64).
template <int kWidth>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
    for (int m = 1; m < kWidth; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
    return x;
}

// f32 append: copy one row of one live head.  block 64, each lane 2 channels.
__global__ __launch_bounds__(64) void k_append_f32(const AppendArgs a) {
    const int r = blockIdx.x, j = blockIdx.y, gl = blockIdx.z;
    const int g = arg_byte(a.live_head, gl);
    const int lane = threadIdx.x;
    const size_t src = ((size_t)(a.src_row0[j] + r) * a.n_kv_heads + g) * kHD + 2 * lane;
    const size_t dst = (((size_t)a.seq[j] * a.n_live + gl) * a.capacity + a.dst_row0[j] + r) * kHD
                       + 2 * lane;
    *(float2*)(a.k + dst) = *(const float2*)(a.k_new + src);
    *(float2*)(a.v + dst) = *(const float2*)(a.v_new + src);
}

// q8 append ([P1] quant_row against the field, or against nothing before the
// freeze).  block 128: wave 0 quantises the K row (4 groups of 32 channels,
// 16 lanes per group), wave 1 the V row (one group of 128).
__global__ __launch_bounds__(128) void k_append_q8(const AppendArgs a) {
    const int r = blockIdx.x, j = blockIdx.y, gl = blockIdx.z;
    const int g = arg_byte(a.live_head, gl);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const bool is_k = (wave == 0);
    const size_t src = ((size_t)(a.src_row0[j] + r) * a.n_kv_heads + g) * kHD + 2 * lane;
    const size_t hrow = ((size_t)a.seq[j] * a.n_live + gl) * a.capacity + a.dst_row0[j] + r;
    const float2 x = *(const float2*)((is_k ? a.k_new : a.v_new) + src);
    float r0 = x.x, r1 = x.y;
    if (a.frozen[j]) {
        const float* col = (is_k ? a.kcol : a.vcol) + ((size_t)a.seq[j] * a.n_live + gl) * kHD;
        r0 = __fdiv_rn(r0, col[2 * lane]);
        r1 = __fdiv_rn(r1, col[2 * lane + 1]);
    }
    float am = fmaxf(fabsf(r0), fabsf(r1));
    am = is_k ? group_max<16>(am) : group_max<64>(am);
    const float s = group_scale(am);
    char2 c;
    c.x = quant_code(r0, s);
    c.y = quant_code(r1, s);
    if (is_k)
        *(char2*)(a.kq + ((size_t)a.seq[j] * a.n_live + gl) * kq_rows(a.capacity) * kHD +
                  kq_offset(a.dst_row0[j] + r, 2 * lane)) = c;
    else
        *(char2*)(a.vq + hrow * kHD + 2 * lane) = c;
    if (is_k) {
        if ((lane & 15) == 0) a.ks[hrow * kKScales + (lane >> 4)] = s;
    } else {
        if (lane == 0) a.vs[hrow] = s;
    }
}

// Per-row int8 append ([P3] quantize_row_i8).  block 128: wave 0 quantises
// the K row, wave 1 the V row; lane holds 2 channels.  scale = max|x| / 127
// (1 for a zero row), code = clamp(round_ties_even(x / scale), -127, 127).
__global__ __launch_bounds__(128) void k_append_i8(const AppendArgs a) {
    const int r = blockIdx.x, j = blockIdx.y, gl = blockIdx.z;
    const int g = arg_byte(a.live_head, gl);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const bool is_k = (wave == 0);
    const size_t src = ((size_t)(a.src_row0[j] + r) * a.n_kv_heads + g) * kHD + 2 * lane;
    const size_t hrow = ((size_t)a.seq[j] * a.n_live + gl) * a.capacity + a.dst_row0[j] + r;
    const float2 x = *(const float2*)((is_k ? a.k_new : a.v_new) + src);
    const float am = group_max<64>(fmaxf(fabsf(x.x), fabsf(x.y)));
    const float s = am > 0.0f ? __fdiv_rn(am, 127.0f) : 1.0f;
    const float c0 = fminf(fmaxf(rintf(__fdiv_rn(x.x, s)), -127.0f), 127.0f);
    const float c1 = fminf(fmaxf(rintf(__fdiv_rn(x.y, s)), -127.0f), 127.0f);
    char2 c;
    c.x = (int8_t)(int)c0;
    c.y = (int8_t)(int)c1;
    if (is_k)
        *(char2*)(a.kq + ((size_t)a.seq[j] * a.n_live + gl) * kq_rows(a.capacity) * kHD +
                  kq_offset(a.dst_row0[j] + r, 2 * lane)) = c;
    else
        *(char2*)(a.vq + hrow * kHD + 2 * lane) = c;
    if (lane == 0) (is_k ? a.ks : a.vs)[hrow] = s;
}

// Freeze + requantise ([P1] freeze_cols) for one (sequence, live head), one
// block of kFreezeThreads.  The stored rows are staged in LDS kFreezeRows at a
// time (K codes in their tile-major order, the K scale records, V codes, V
// scales) with 16-byte loads.  Threads 0..127 own the K channels and 128..255
// the V channels for the RMS sum, which runs over the rows in order, multiply
// then add, exactly as the page's loop does per channel.  Once the field is
// known every row is requantised on its own: wave w takes rows w, w + 16, ..
// of the chunk, lane l channels 2 l and 2 l + 1, the K group max over 16
// lanes and the V row max over the wave.
constexpr int kFreezeRows = 64;
constexpr int kFreezeThreads = 1024;

__global__ __launch_bounds__(kFreezeThreads) void k_freeze(const FreezeArgs a) {
    __shared__ __attribute__((aligned(16))) int8_t s_kq[kFreezeRows * kHD];
    __shared__ __attribute__((aligned(16))) int8_t s_vq[kFreezeRows * kHD];
    __shared__ __attribute__((aligned(16))) float s_ks[kFreezeRows * kKScales];
    __shared__ float s_vs[kFreezeRows];
    __shared__ float s_col[2 * kHD];
    const int gl = blockIdx.x, j = blockIdx.y;
    const int b = a.seq[j], n = a.n[j];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    constexpr int kWavesF = kFreezeThreads / 64;
    const size_t head = (size_t)b * a.n_live + gl;
    const size_t row0 = head * a.capacity;
    int8_t* KQ = a.kq + head * kq_rows(a.capacity) * kHD;    // tile-major K codes
    float* KS = a.ks + row0 * kKScales;
    int8_t* VQ = a.vq + row0 * kHD;
    float* VS = a.vs + row0;

    // rows [p0, p0 + m) into LDS (p0 a multiple of kFreezeRows; the K tile
    // holding the last row is whole in storage)
    auto stage = [&](int p0, int m) {
        const int m16 = (m + kTileRows - 1) & ~(kTileRows - 1);
        for (int i = tid; i < m16 * kHD / 16; i += kFreezeThreads)
            *(uint4*)(s_kq + 16 * i) = *(const uint4*)(KQ + (size_t)p0 * kHD + 16 * i);
        for (int i = tid; i < m * kHD / 16; i += kFreezeThreads)
            *(uint4*)(s_vq + 16 * i) = *(const uint4*)(VQ + (size_t)p0 * kHD + 16 * i);
        for (int i = tid; i < m; i += kFreezeThreads) {
            *(float4*)(s_ks + kKScales * i) = *(const float4*)(KS + (size_t)(p0 + i) * kKScales);
            s_vs[i] = VS[p0 + i];
        }
    };

    // ---- the RMS of each channel over the n stored rows, in row order ----
    const bool is_k = tid < kHD;
    const int d = tid & (kHD - 1);
    float acc = 0.0f;
    for (int p0 = 0; p0 < n; p0 += kFreezeRows) {
        const int m = min(kFreezeRows, n - p0);
        if (p0 > 0) __syncthreads();                   // the previous chunk is summed
        stage(p0, m);
        __syncthreads();
        if (tid < 2 * kHD) {
            for (int p = 0; p < m; ++p) {
                const float x = is_k ? (float)s_kq[kq_offset(p, d)] * s_ks[kKScales * p + d / kKGroup]
                                     : (float)s_vq[p * kHD + d] * s_vs[p];
                const float sq = x * x;
                acc = acc + sq;
            }
        }
    }
    if (tid < 2 * kHD) {
        const float col = fmaxf(sqrtf(__fdiv_rn(acc, (float)n)), 1e-6f);
        (is_k ? a.kcol : a.vcol)[head * kHD + d] = col;
        s_col[tid] = col;
    }

    // ---- every row requantised against the field (rows are independent) ----
    for (int p0 = 0; p0 < n; p0 += kFreezeRows) {
        const int m = min(kFreezeRows, n - p0);
        __syncthreads();                               // s_col written; the previous chunk is done
        if (n > kFreezeRows) {                         // otherwise the only chunk is still staged
            stage(p0, m);
            __syncthreads();
        }
        const int c = 2 * lane;
        for (int p = wave; p < m; p += kWavesF) {
            // K: groups of 32 channels (16 lanes)
            const char2 kc = *(const char2*)(s_kq + kq_offset(p, c));
            const float ksc = s_ks[kKScales * p + c / kKGroup];
            const float r0 = __fdiv_rn((float)kc.x * ksc, s_col[c]);
            const float r1 = __fdiv_rn((float)kc.y * ksc, s_col[c + 1]);
            const float sk = group_scale(group_max<16>(fmaxf(fabsf(r0), fabsf(r1))));
            char2 qk;
            qk.x = quant_code(r0, sk);
            qk.y = quant_code(r1, sk);
            *(char2*)(KQ + kq_offset(p0 + p, c)) = qk;
            if ((lane & 15) == 0) KS[(size_t)(p0 + p) * kKScales + lane / 16] = sk;
            // V: one group of 128 channels (the wave)
            const char2 vc = *(const char2*)(s_vq + p * kHD + c);
            const float vsc = s_vs[p];
            const float v0 = __fdiv_rn((float)vc.x * vsc, s_col[kHD + c]);
            const float v1 = __fdiv_rn((float)vc.y * vsc, s_col[kHD + c + 1]);
            const float sv = group_scale(group_max<64>(fmaxf(fabsf(v0), fabsf(v1))));
            char2 qv;
            qv.x = quant_code(v0, sv);
            qv.y = quant_code(v1, sv);
            *(char2*)(VQ + (size_t)(p0 + p) * kHD + c) = qv;
            if (lane == 0) VS[p0 + p] = sv;
        }
    }
}

// Front-trim moves ([P2] trim_window: the kept rows move to the front,
// unchanged and in order), one round per launch for every sequence listed in it: rows [src,
// src + m) go to [dst, dst + m) with src - dst = d >= m, so a launch's source
// and destination never overlap, and consecutive launches on the stream order
// a round's reads before the next round's writes.  grid (blocks, sequence x
// live head, buffer), block 256, a grid-stride loop of 16-byte copies (4-byte
// for the one-per-row scales: vs, and ks of the per-row int8 kind).
template <class T>
__device__ __forceinline__ void copy_rows(T* base, int units_per_row, int src, int dst, int m) {
    const T* s = base + (size_t)src * units_per_row;
    T* d = base + (size_t)dst * units_per_row;
    const size_t n = (size_t)m * units_per_row;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        d[i] = s[i];
}

// K codes, tile-major: threads walk the destination's 16-byte pieces (row,
// 16 channels) in storage order over the 16-row tiles that hold rows
// [dst, dst + m), so a wave writes 1 KB runs; pieces of rows outside the
// range are skipped.  Each piece comes from the source row at the same
// offset in [src, src + m).
__device__ __forceinline__ void copy_kq_rows(int8_t* base, int src, int dst, int m) {
    const int db = dst & ~(kTileRows - 1);
    const size_t n = (size_t)((dst + m - db + kTileRows - 1) / kTileRows) * (kTileRows * kHD / 16);
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const int r = db + kTileRows * (int)(i >> 7) + (int)(i & 15);
        const int c = 16 * (int)((i >> 4) & 7);
        if (r < dst || r >= dst + m) continue;
        *(uint4*)(base + kq_offset(r, c)) = *(const uint4*)(base + kq_offset(r - dst + src, c));
    }
}

__global__ __launch_bounds__(256) void k_move_chunk(const MoveArgs a) {
    const int j = blockIdx.y / a.n_live, gl = blockIdx.y - j * a.n_live;
    const int src = a.src[j], dst = a.dst[j], m = a.m[j];
    const size_t head = (size_t)a.seq[j] * a.n_live + gl;
    const size_t row0 = head * a.capacity;
    const int z = blockIdx.z;
    const int which = a.kind == KVQ_KIND_F32 ? 4 + z : (a.kind == KVQ_KIND_I8 && z == 1) ? 6 : z;
    switch (which) {
        case 0: copy_kq_rows(a.kq + head * kq_rows(a.capacity) * kHD, src, dst, m); break;
        case 1: copy_rows(reinterpret_cast<uint4*>(a.ks + row0 * kKScales), 1, src, dst, m); break;
        case 2: copy_rows(reinterpret_cast<uint4*>(a.vq + row0 * kHD), kHD / 16, src, dst, m); break;
        case 3: copy_rows(reinterpret_cast<uint32_t*>(a.vs + row0), 1, src, dst, m); break;
        case 4: copy_rows(reinterpret_cast<uint4*>(a.k + row0 * kHD), kHD / 4, src, dst, m); break;
        case 5: copy_rows(reinterpret_cast<uint4*>(a.v + row0 * kHD), kHD / 4, src, dst, m); break;
        default: copy_rows(reinterpret_cast<uint32_t*>(a.ks + row0), 1, src, dst, m); break;
    }
}

}  // namespace

hipError_t launch_trim_moves(const MoveArgs& args, const TrimMove* moves, int count, hipStream_t s) {
    const bool f32 = args.kind == KVQ_KIND_F32;
    for (int r = 0;; ++r) {                            // round r moves rows [r d, r d + m) of each sequence
        bool any = false;
        int i = 0;
        while (i < count) {
            MoveArgs a = args;
            a.n_seq = 0;
            int mmax = 0;
            for (; i < count && a.n_seq < kSeqPerLaunch; ++i) {
                const TrimMove& mv = moves[i];
                const int64_t at = (int64_t)r * mv.d;
                if (mv.d <= 0 || at >= mv.keep) continue;
                const int m = (int)std::min<int64_t>(mv.d, mv.keep - at);
                a.seq[a.n_seq] = mv.seq;
                a.src[a.n_seq] = (int)(at + mv.d);
                a.dst[a.n_seq] = (int)at;
                a.m[a.n_seq] = m;
                ++a.n_seq;
                mmax = std::max(mmax, m);
            }
            if (a.n_seq == 0) continue;
            any = true;
            const size_t units = (size_t)mmax * (f32 ? kHD / 4 : kHD / 16);   // largest buffer, 16-byte units
            const size_t want = (units + 1023) / 1024;
            const int blocks = (int)(want < 128 ? want : 128);
            hipLaunchKernelGGL(k_move_chunk, dim3(blocks, a.n_live * a.n_seq, f32 ? 2 : 4), dim3(256), 0, s, a);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (!any) return hipSuccess;
    }
}

hipError_t launch_append_f32(const AppendArgs& a, int n_rows, hipStream_t s) {
    hipLaunchKernelGGL(k_append_f32, dim3(n_rows, a.n_seq, a.n_live), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_append_q8(const AppendArgs& a, int n_rows, hipStream_t s) {
    hipLaunchKernelGGL(k_append_q8, dim3(n_rows, a.n_seq, a.n_live), dim3(128), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_append_i8(const AppendArgs& a, int n_rows, hipStream_t s) {
    hipLaunchKernelGGL(k_append_i8, dim3(n_rows, a.n_seq, a.n_live), dim3(128), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_freeze(const FreezeArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_freeze, dim3(a.n_live, a.n_seq), dim3(kFreezeThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
