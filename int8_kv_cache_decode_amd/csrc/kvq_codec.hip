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
    const int g = a.live_head[gl];
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
    const int g = a.live_head[gl];
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
    const int g = a.live_head[gl];
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

// Freeze + requantise ([P1] freeze_cols) for one (sequence, live head).
// block 128: thread d owns channel d.  The RMS sum runs over the rows in
// order, multiply then add, exactly as the page's loop does per channel.
__global__ __launch_bounds__(128) void k_freeze(const FreezeArgs a) {
    __shared__ float red[2][2];
    const int gl = blockIdx.x, j = blockIdx.y;
    const int b = a.seq[j], n = a.n[j];
    const int d = threadIdx.x, wave = d >> 6, lane = d & 63;
    const size_t head = (size_t)b * a.n_live + gl;
    const size_t row0 = head * a.capacity;

    // ---- K: group of 32 channels, scale per (row, group) ----
    {
        int8_t* q = a.kq + head * kq_rows(a.capacity) * kHD;    // tile-major K codes
        float* s = a.ks + row0 * kKScales;
        float acc = 0.0f;
        for (int p = 0; p < n; ++p) {
            const float x = (float)q[kq_offset(p, d)] * s[(size_t)p * kKScales + d / kKGroup];
            const float sq = x * x;
            acc = acc + sq;
        }
        const float col = fmaxf(sqrtf(__fdiv_rn(acc, (float)n)), 1e-6f);
        a.kcol[head * kHD + d] = col;
        for (int p = 0; p < n; ++p) {
            const float x = (float)q[kq_offset(p, d)] * s[(size_t)p * kKScales + d / kKGroup];
            const float r = __fdiv_rn(x, col);
            const float sc = group_scale(group_max<32>(fabsf(r)));
            q[kq_offset(p, d)] = quant_code(r, sc);
            if ((d & (kKGroup - 1)) == 0) s[(size_t)p * kKScales + d / kKGroup] = sc;
        }
    }
    // ---- V: one group of 128 channels, scale per row ----
    {
        int8_t* q = a.vq + row0 * kHD;
        float* s = a.vs + row0;
        float acc = 0.0f;
        for (int p = 0; p < n; ++p) {
            const float x = (float)q[(size_t)p * kHD + d] * s[p];
            const float sq = x * x;
            acc = acc + sq;
        }
        const float col = fmaxf(sqrtf(__fdiv_rn(acc, (float)n)), 1e-6f);
        a.vcol[head * kHD + d] = col;
        for (int p = 0; p < n; ++p) {
            const float x = (float)q[(size_t)p * kHD + d] * s[p];
            const float r = __fdiv_rn(x, col);
            const float wm = group_max<64>(fabsf(r));
            if (lane == 0) red[p & 1][wave] = wm;
            __syncthreads();                       // every thread has read s[p]
            const float sc = group_scale(fmaxf(red[p & 1][0], red[p & 1][1]));
            q[(size_t)p * kHD + d] = quant_code(r, sc);
            if (d == 0) s[p] = sc;
        }
    }
}

// Front-trim move ([P2] trim_window: the rows that stay keep their order and
// values), one chunk of m <= d rows per launch: rows [src, src + m) go to
// [dst, dst + m) with src - dst = d >= m, so a launch's source and
// destination never overlap, and consecutive launches on the stream order a
// chunk's reads before the next chunk's writes.  grid (blocks, live head,
// buffer), block 256, a grid-stride loop of 16-byte copies (4-byte for the
// one-per-row scales: vs, and ks of the per-row int8 kind).
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

__global__ __launch_bounds__(256) void k_move_chunk(const MoveArgs a, int src, int dst, int m) {
    const size_t head = (size_t)a.seq * a.n_live + blockIdx.y;
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

hipError_t launch_move_rows(const MoveArgs& a, hipStream_t s) {
    for (int r = 0; r < a.keep; r += a.d) {
        const int m = min(a.d, a.keep - r);
        const bool f32 = a.kind == KVQ_KIND_F32;
        const size_t units = (size_t)m * (f32 ? kHD / 4 : kHD / 16);     // largest buffer, 16-byte units
        const size_t want = (units + 1023) / 1024;
        const int blocks = (int)(want < 128 ? want : 128);
        hipLaunchKernelGGL(k_move_chunk, dim3(blocks, a.n_live, f32 ? 2 : 4), dim3(256), 0, s, a, a.d + r, r, m);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
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
    hipLaunchKernelGGL(k_freeze, dim3(a.n_live, a.n_seq), dim3(128), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
