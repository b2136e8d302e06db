// kvq_api.hip -- the C ABI declared in include/kvq.h: host-side validation,
// work partitioning and kernel launches.  Every check runs before anything
// is enqueued, so a refused call leaves the cache untouched ([P3]
// franken_ocr 0.8.0 rswa.rs: malformed steps are refused before any K/V
// write; record_prefill / write_decode_step validate first).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "kvq_internal.h"

using namespace kvq;

namespace {

thread_local std::string g_err;

// Workspace of decode_attn_q8_noalloc: the partial softmax states of the
// split decode live in this device array instead of a caller's buffer.  Each
// GPU the library runs on holds its own copy until the process ends.  Host
// code never passes `scratch` itself to a kernel (on the host it names a
// stand-in, not device memory): it uses the address scratch_address()
// looked up for the current device.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; null on a runtime error.
void* scratch_address() {
    constexpr int kDevices = 64;
    static std::mutex mu;
    static void* addr[kDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Geometry checks shared by every call; `kind` 0 accepts either kind.
int check_cache(const kvq_cache* c, int kind, const char* fn) {
    if (!c) return fail(KVQ_EINVAL, "%s: null cache", fn);
    if (c->head_dim != KVQ_HEAD_DIM) return fail(KVQ_EINVAL, "%s: head_dim %d != 128", fn, c->head_dim);
    if (c->batch < 1 || c->capacity < 1 || c->capacity > KVQ_MAX_CAPACITY)
        return fail(KVQ_EINVAL, "%s: batch %d must be >= 1, capacity %d within 1..%d", fn, c->batch, c->capacity,
                    KVQ_MAX_CAPACITY);
    if (c->n_kv_heads < 1 || c->n_kv_heads > KVQ_MAX_KV_HEADS)
        return fail(KVQ_EINVAL, "%s: n_kv_heads %d outside 1..%d", fn, c->n_kv_heads, KVQ_MAX_KV_HEADS);
    int live = 0;
    for (int g = 0; g < c->n_kv_heads; ++g) {
        if (c->live_slot[g] >= 0) {
            if (c->live_slot[g] != live) return fail(KVQ_EINVAL, "%s: live_slot table is not dense", fn);
            ++live;
        }
    }
    if (live != c->n_live) return fail(KVQ_EINVAL, "%s: n_live %d does not match live_slot", fn, c->n_live);
    if (!c->len || !c->frozen) return fail(KVQ_EINVAL, "%s: null host len/frozen arrays", fn);
    if (kind && c->kind != kind)
        return fail(KVQ_ESTATE, "%s: cache kind %d, this call needs kind %d", fn, c->kind, kind);
    if (c->kind == KVQ_KIND_F32) {
        if (!c->k || !c->v) return fail(KVQ_EINVAL, "%s: f32 cache without k/v buffers", fn);
        if (!aligned16(c->k) || !aligned16(c->v)) return fail(KVQ_EINVAL, "%s: k/v not 16-byte aligned", fn);
    } else if (c->kind == KVQ_KIND_Q8) {
        if (!c->kq || !c->ks || !c->vq || !c->vs || !c->kcol || !c->vcol)
            return fail(KVQ_EINVAL, "%s: q8 cache with a missing buffer", fn);
        if (!aligned16(c->kq) || !aligned16(c->ks) || !aligned16(c->vq) || !aligned16(c->vs) ||
            !aligned16(c->kcol) || !aligned16(c->vcol))
            return fail(KVQ_EINVAL, "%s: q8 buffers not 16-byte aligned", fn);
    } else if (c->kind == KVQ_KIND_I8) {
        if (!c->kq || !c->ks || !c->vq || !c->vs) return fail(KVQ_EINVAL, "%s: i8 cache with a missing buffer", fn);
        if (!aligned16(c->kq) || !aligned16(c->ks) || !aligned16(c->vq) || !aligned16(c->vs))
            return fail(KVQ_EINVAL, "%s: i8 buffers not 16-byte aligned", fn);
    } else {
        return fail(KVQ_EINVAL, "%s: unknown cache kind %d", fn, c->kind);
    }
    for (int b = 0; b < c->batch; ++b)
        if (c->len[b] < 0 || c->len[b] > c->capacity)
            return fail(KVQ_ESTATE, "%s: len[%d] = %d outside 0..capacity", fn, b, c->len[b]);
    return KVQ_OK;
}

void fill_live(const kvq_cache* c, int8_t* live_head) {
    for (int g = 0; g < c->n_kv_heads; ++g)
        if (c->live_slot[g] >= 0) live_head[c->live_slot[g]] = (int8_t)g;
}

int device_status(hipError_t e, const char* fn) {
    if (e != hipSuccess) return fail(KVQ_EDEVICE, "%s: %s", fn, hipGetErrorString(e));
    return KVQ_OK;
}

// ---- append ---------------------------------------------------------------
struct Seg {
    int seq, src_row0, dst_row0, n;
    bool frozen;
};

AppendArgs base_append(const kvq_cache* c, const float* k_new, const float* v_new) {
    AppendArgs a;
    memset(&a, 0, sizeof a);
    a.k_new = k_new;
    a.v_new = v_new;
    a.k = c->k;
    a.v = c->v;
    a.kq = c->kq;
    a.ks = c->ks;
    a.vq = c->vq;
    a.vs = c->vs;
    a.kcol = c->kcol;
    a.vcol = c->vcol;
    a.n_kv_heads = c->n_kv_heads;
    a.n_live = c->n_live;
    a.capacity = c->capacity;
    fill_live(c, a.live_head);
    return a;
}

// R-SWA caches: f32, or the per-row int8 kind ([P3] keeps its int8 mirror
// in the same reference + ring layout).
int check_ring_cache(const kvq_cache* c, const char* fn) {
    const int rc = check_cache(c, 0, fn);
    if (rc) return rc;
    if (c->kind != KVQ_KIND_F32 && c->kind != KVQ_KIND_I8)
        return fail(KVQ_ESTATE, "%s: R-SWA needs an f32 or i8 cache (kind %d)", fn, c->kind);
    return KVQ_OK;
}

// Launch equal-length segments (same n) in batches of kSeqPerLaunch, with
// the append kernel of the cache's own kind (the caller has checked it, so
// every buffer that kernel writes is present).
int launch_segments(const kvq_cache* c, const float* k_new, const float* v_new,
                    const std::vector<Seg>& segs, hipStream_t s, const char* fn) {
    if (c->n_live == 0) return KVQ_OK;
    const int kind = c->kind;
    if (kind != KVQ_KIND_F32 && kind != KVQ_KIND_Q8 && kind != KVQ_KIND_I8)
        return fail(KVQ_EINVAL, "%s: unknown cache kind %d", fn, kind);
    size_t i = 0;
    while (i < segs.size()) {
        AppendArgs a = base_append(c, k_new, v_new);
        const int n = segs[i].n;
        int ns = 0;
        while (i < segs.size() && ns < kSeqPerLaunch && segs[i].n == n) {
            a.seq[ns] = segs[i].seq;
            a.src_row0[ns] = segs[i].src_row0;
            a.dst_row0[ns] = segs[i].dst_row0;
            a.frozen[ns] = segs[i].frozen ? 1 : 0;
            ++ns;
            ++i;
        }
        a.n_seq = ns;
        if (n == 0) continue;
        const int rc = device_status(kind == KVQ_KIND_Q8   ? launch_append_q8(a, n, s)
                                     : kind == KVQ_KIND_I8 ? launch_append_i8(a, n, s)
                                                           : launch_append_f32(a, n, s),
                                     fn);
        if (rc) return rc;
    }
    return KVQ_OK;
}

int launch_freeze_list(const kvq_cache* c, const std::vector<std::pair<int, int>>& list,
                       hipStream_t s, const char* fn) {
    if (c->n_live == 0) return KVQ_OK;
    for (size_t i = 0; i < list.size(); i += kSeqPerLaunch) {
        FreezeArgs f;
        memset(&f, 0, sizeof f);
        f.kq = c->kq;
        f.ks = c->ks;
        f.vq = c->vq;
        f.vs = c->vs;
        f.kcol = c->kcol;
        f.vcol = c->vcol;
        f.n_live = c->n_live;
        f.capacity = c->capacity;
        f.n_seq = (int)std::min<size_t>(kSeqPerLaunch, list.size() - i);
        for (int j = 0; j < f.n_seq; ++j) {
            f.seq[j] = list[i + j].first;
            f.n[j] = list[i + j].second;
        }
        const int rc = device_status(launch_freeze(f, s), fn);
        if (rc) return rc;
    }
    return KVQ_OK;
}

int check_append_args(const kvq_cache* c, int seq, int n_rows, const float* k_new,
                      const float* v_new, const char* fn) {
    if (seq == KVQ_ALL_SEQS) {
        if (n_rows != 1) return fail(KVQ_EINVAL, "%s: seq=ALL appends exactly one row (n_rows=%d)", fn, n_rows);
        for (int b = 0; b < c->batch; ++b)
            if (c->len[b] + 1 > c->capacity)
                return fail(KVQ_ECAPACITY, "%s: sequence %d is full (len %d, capacity %d)", fn, b, c->len[b], c->capacity);
    } else {
        if (seq < 0 || seq >= c->batch) return fail(KVQ_EINVAL, "%s: seq %d outside 0..%d", fn, seq, c->batch - 1);
        if (n_rows < 0) return fail(KVQ_EINVAL, "%s: n_rows %d < 0", fn, n_rows);
        if ((int64_t)c->len[seq] + n_rows > c->capacity)
            return fail(KVQ_ECAPACITY, "%s: len %d + n_rows %d exceeds capacity %d", fn, c->len[seq], n_rows, c->capacity);
    }
    if (n_rows > 0 && (!k_new || !v_new)) return fail(KVQ_EINVAL, "%s: null k_new/v_new", fn);
    if (n_rows > 0 && (!aligned16(k_new) || !aligned16(v_new)))
        return fail(KVQ_EINVAL, "%s: k_new/v_new not 16-byte aligned", fn);
    return KVQ_OK;
}

// ---- decode ---------------------------------------------------------------
size_t ws_slots(const kvq_cache* c) { return max_slots(std::min(c->batch, kSeqPerLaunch), c->n_live); }

size_t ws_need(const kvq_cache* c, int hpk) {
    const size_t slots = ws_slots(c);
    size_t bytes = slots * hpk * kHD * sizeof(float) + slots * hpk * 2 * sizeof(float);
    return (bytes + 255) & ~(size_t)255;
}

int check_decode_args(const kvq_cache* c, int n_q_heads, const float* q, float* out,
                      void* ws, size_t ws_bytes, const char* fn, int* hpk_out) {
    if (n_q_heads < 1 || n_q_heads % c->n_kv_heads != 0)
        return fail(KVQ_EINVAL, "%s: n_q_heads %d is not a multiple of n_kv_heads %d", fn, n_q_heads, c->n_kv_heads);
    const int hpk = n_q_heads / c->n_kv_heads;
    if (hpk != 1 && hpk != 2 && hpk != 4 && hpk != 8)
        return fail(KVQ_EINVAL, "%s: group size %d not in {1,2,4,8}", fn, hpk);
    if (!q || !out) return fail(KVQ_EINVAL, "%s: null q/out", fn);
    if (!aligned16(q) || !aligned16(out)) return fail(KVQ_EINVAL, "%s: q/out not 16-byte aligned", fn);
    if (!ws) return fail(KVQ_EINVAL, "%s: null workspace", fn);
    if (!aligned16(ws)) return fail(KVQ_EINVAL, "%s: workspace not 16-byte aligned", fn);
    const size_t need = ws_need(c, hpk);
    if (ws_bytes < need) return fail(KVQ_EINVAL, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    *hpk_out = hpk;
    return KVQ_OK;
}

// Options of the _ex calls: first[b] >= 0, softcap finite and >= 0.
int check_decode_opts(const kvq_cache* c, const kvq_decode_opts* o, const char* fn) {
    if (!o) return KVQ_OK;
    if (o->reserved != 0) return fail(KVQ_EINVAL, "%s: opts.reserved must be 0", fn);
    if (!(o->softcap >= 0.0f) || std::isinf(o->softcap))
        return fail(KVQ_EINVAL, "%s: softcap %g must be finite and >= 0", fn, (double)o->softcap);
    if (o->first)
        for (int b = 0; b < c->batch; ++b)
            if (o->first[b] < 0) return fail(KVQ_EINVAL, "%s: first[%d] = %d < 0", fn, b, o->first[b]);
    return KVQ_OK;
}

// Partition and launch one decode over every sequence.  lens: rows stored
// per sequence; wrows: R-SWA row fed from k_new/v_new (or null); opts: the
// visible-row start, soft-cap and sinks (or null).
int run_decode(const kvq_cache* c, int n_q_heads, int hpk, const float* q, float* out, void* ws,
               const int32_t* lens, const int32_t* wrows, const float* k_new, const float* v_new,
               const kvq_decode_opts* opts, hipStream_t s, const char* fn) {
    DecodeArgs a;
    memset(&a, 0, sizeof a);
    a.q = q;
    a.out = out;
    a.k = c->k;
    a.v = c->v;
    a.kq = c->kq;
    a.ks = c->ks;
    a.vq = c->vq;
    a.vs = c->vs;
    a.kcol = c->kcol;
    a.vcol = c->vcol;
    a.ws_acc = (float*)ws;
    a.ws_ml = (float*)ws + ws_slots(c) * hpk * kHD;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_store = c->k;
    a.v_store = c->v;
    a.kq_store = c->kq;
    a.ks_store = c->ks;
    a.vq_store = c->vq;
    a.vs_store = c->vs;
    a.n_kv_heads = c->n_kv_heads;
    a.n_live = c->n_live;
    a.n_q_heads = n_q_heads;
    a.hpk = hpk;
    a.capacity = c->capacity;
    a.softcap2 = (opts && opts->softcap > 0.0f) ? (double)opts->softcap * 1.4426950408889634 : 0.0;
    a.sinks = opts ? opts->sinks : nullptr;
    fill_live(c, a.live_head);
    memcpy(a.live_slot, c->live_slot, sizeof a.live_slot);
    for (int s0 = 0; s0 < c->batch; s0 += kSeqPerLaunch) {
        const int ns = std::min(kSeqPerLaunch, c->batch - s0);
        a.seq0 = s0;
        a.n_seq = ns;
        int64_t tiles = 0;
        for (int j = 0; j < ns; ++j) {
            const int L = lens[s0 + j];
            // [P2] attend_group_upto: first clamped so that one row stays visible
            const int f = (opts && opts->first && L > 0) ? std::min(opts->first[s0 + j], L - 1) : 0;
            a.len[j] = L;
            // int8 kinds: the tile stream starts on a K tile boundary
            const int st = c->kind == KVQ_KIND_F32 ? f : f & ~(kTileRows - 1);
            a.first[j] = f;
            a.start[j] = st;
            a.ntile[j] = (L - st + kTileRows - 1) / kTileRows;
            a.wrow[j] = wrows ? wrows[s0 + j] : -1;
            a.frozen[j] = c->frozen[s0 + j] ? 1 : 0;
            a.tile_base[j] = (int32_t)tiles;
            tiles += (int64_t)a.ntile[j] * c->n_live;
            // unreachable with real memory sizes (2^31 tiles of q8 rows > 9 TB)
            if (tiles >= ((int64_t)1 << 31))
                return fail(KVQ_EINVAL, "%s: more than 2^31 tiles in one launch", fn);
        }
        a.tile_base[ns] = (int32_t)tiles;
        a.n_tiles = (int)tiles;
        const hipError_t e = c->kind == KVQ_KIND_Q8   ? launch_decode_q8(a, s)
                             : c->kind == KVQ_KIND_I8 ? launch_decode_i8(a, s)
                                                      : launch_decode_f32(a, s);
        const int rc = device_status(e, fn);
        if (rc) return rc;
    }
    return KVQ_OK;
}

// [P3] RingCache::checkpoint: the cursors of one ring.
void take_checkpoint(const kvq_cache* c, const kvq_ring& r, int seq, int stream, kvq_ring_checkpoint* cp) {
    cp->cache = c;
    cp->seq = seq;
    cp->prefill_len = r.prefill_len;
    cp->ring_len = r.ring_len;
    cp->ring_pos = r.ring_pos;
    cp->epoch = r.epoch;
    cp->stream = stream;
    cp->writes = r.writes;
}

// [P3] RingCache::rollback_to on one ring whose checkpoint identity the
// caller has checked: the page's refusals, in its order, before any change;
// then the cursors are restored, and a rollback that discards writes starts
// a new lineage.
int rollback_ring(kvq_ring& r, const kvq_ring_checkpoint* cp, const char* fn) {
    if (cp->prefill_len != r.prefill_len)
        return fail(KVQ_ESTATE, "%s: checkpoint prefill_len %d != %d", fn, cp->prefill_len, r.prefill_len);
    if (cp->epoch != r.epoch)
        return fail(KVQ_ESTATE, "%s: stale checkpoint lineage (epoch %d != %d)", fn, cp->epoch, r.epoch);
    if (cp->writes > r.writes)
        return fail(KVQ_ESTATE, "%s: checkpoint is from the future (writes %lld > %lld)", fn, (long long)cp->writes,
                    (long long)r.writes);
    const int64_t discarded = r.writes - cp->writes;
    if (cp->ring_len < 0 || cp->ring_len > KVQ_RING_WINDOW || discarded > KVQ_RING_WINDOW - cp->ring_len)
        return fail(KVQ_ESTATE, "%s: not lossless: %lld discarded writes wrapped the ring past ring_len %d", fn,
                    (long long)discarded, cp->ring_len);
    if (cp->ring_pos < 0 || cp->ring_pos >= KVQ_RING_WINDOW)
        return fail(KVQ_ESTATE, "%s: checkpoint ring_pos %d outside 0..%d", fn, cp->ring_pos, KVQ_RING_WINDOW - 1);
    if (discarded > 0 && r.epoch == INT32_MAX) return fail(KVQ_ESTATE, "%s: lineage epoch exhausted", fn);
    r.ring_len = cp->ring_len;
    r.ring_pos = cp->ring_pos;
    r.writes = cp->writes;
    if (discarded > 0) r.epoch += 1;
    return KVQ_OK;
}

// A shared group's stream s: the cache kind, the indices, and a group that
// is recorded on sequence seq with n_streams rings.
int check_shared_stream(const kvq_cache* c, int seq, const kvq_ring* rings, int n_streams, int s, const char* fn) {
    const int rc = check_ring_cache(c, fn);
    if (rc) return rc;
    if (!rings) return fail(KVQ_EINVAL, "%s: null rings", fn);
    if (seq < 0 || seq >= c->batch) return fail(KVQ_EINVAL, "%s: seq %d outside 0..%d", fn, seq, c->batch - 1);
    if (n_streams < 1 || n_streams > kVerifyMaxQ)
        return fail(KVQ_EINVAL, "%s: n_streams %d outside 1..%d", fn, n_streams, kVerifyMaxQ);
    if (s < 0 || s >= n_streams) return fail(KVQ_EINVAL, "%s: stream %d outside 0..%d", fn, s, n_streams - 1);
    const int pre = rings[s].prefill_len;
    if (pre < 0) return fail(KVQ_ESTATE, "%s: stream %d: group not recorded", fn, s);
    if ((int64_t)c->len[seq] != (int64_t)pre + (int64_t)KVQ_RING_WINDOW * n_streams)
        return fail(KVQ_ESTATE, "%s: len %d != prefill %d + %d rings", fn, c->len[seq], pre, n_streams);
    return KVQ_OK;
}

}  // namespace

extern "C" {

int kvq_cache_init(kvq_cache* c, int kind, int batch, int n_kv_heads, int head_dim, int capacity,
                   const uint8_t* alive, int32_t* len_host, uint8_t* frozen_host) {
    const char* fn = "kvq_cache_init";
    if (!c) return fail(KVQ_EINVAL, "%s: null cache", fn);
    if (kind != KVQ_KIND_F32 && kind != KVQ_KIND_Q8 && kind != KVQ_KIND_I8)
        return fail(KVQ_EINVAL, "%s: unknown kind %d", fn, kind);
    if (head_dim != KVQ_HEAD_DIM) return fail(KVQ_EINVAL, "%s: head_dim %d != 128", fn, head_dim);
    if (batch < 1 || capacity < 1 || capacity > KVQ_MAX_CAPACITY)
        return fail(KVQ_EINVAL, "%s: batch must be >= 1 and capacity within 1..%d", fn, KVQ_MAX_CAPACITY);
    if (n_kv_heads < 1 || n_kv_heads > KVQ_MAX_KV_HEADS)
        return fail(KVQ_EINVAL, "%s: n_kv_heads %d outside 1..%d", fn, n_kv_heads, KVQ_MAX_KV_HEADS);
    if (!len_host || !frozen_host) return fail(KVQ_EINVAL, "%s: null len/frozen host arrays", fn);
    memset(c, 0, sizeof *c);
    c->kind = kind;
    c->batch = batch;
    c->n_kv_heads = n_kv_heads;
    c->head_dim = head_dim;
    c->capacity = capacity;
    for (int g = 0; g < KVQ_MAX_KV_HEADS; ++g) c->live_slot[g] = -1;
    int live = 0;
    for (int g = 0; g < n_kv_heads; ++g)
        if (!alive || alive[g]) c->live_slot[g] = (int8_t)live++;
    c->n_live = live;
    c->len = len_host;
    c->frozen = frozen_host;
    for (int b = 0; b < batch; ++b) {
        len_host[b] = 0;
        frozen_host[b] = 0;
    }
    return KVQ_OK;
}

size_t kvq_buffer_bytes(const kvq_cache* c, int which) {
    if (!c || c->head_dim != KVQ_HEAD_DIM || c->batch < 1 || c->capacity < 1) return 0;
    const size_t rows = (size_t)c->batch * c->n_live * c->capacity;
    const size_t heads = (size_t)c->batch * c->n_live;
    const bool f32 = c->kind == KVQ_KIND_F32, q8 = c->kind == KVQ_KIND_Q8, i8 = c->kind == KVQ_KIND_I8;
    switch (which) {
        case KVQ_BUF_K:
        case KVQ_BUF_V: return f32 ? rows * kHD * sizeof(float) : 0;
        case KVQ_BUF_KQ: return (q8 || i8) ? heads * (size_t)kq_rows(c->capacity) * kHD : 0;   // tile-major
        case KVQ_BUF_VQ: return (q8 || i8) ? rows * kHD : 0;
        case KVQ_BUF_KS: return q8 ? rows * kKScales * sizeof(float) : i8 ? rows * sizeof(float) : 0;
        case KVQ_BUF_VS: return (q8 || i8) ? rows * sizeof(float) : 0;
        case KVQ_BUF_KCOL:
        case KVQ_BUF_VCOL: return q8 ? heads * kHD * sizeof(float) : 0;
        default: return 0;
    }
}

size_t kvq_cache_bytes(const kvq_cache* c) {
    if (!c || !c->len || !c->frozen) return 0;
    size_t bytes = 0;
    for (int b = 0; b < c->batch; ++b) {
        const size_t rows = (size_t)c->len[b] * c->n_live;
        if (c->kind == KVQ_KIND_F32) {
            bytes += rows * 2 * kHD * sizeof(float);
        } else if (c->kind == KVQ_KIND_I8) {
            bytes += rows * 2 * (kHD + sizeof(float));
        } else {
            bytes += rows * (kHD + kKScales * sizeof(float) + kHD + sizeof(float));
            if (c->frozen[b]) bytes += (size_t)c->n_live * 2 * kHD * sizeof(float);
        }
    }
    return bytes;
}

int kv_append_f32(kvq_cache* c, int seq, int n_rows, const float* k_new, const float* v_new,
                  void* stream) {
    const char* fn = "kv_append_f32";
    int rc = check_cache(c, KVQ_KIND_F32, fn);
    if (rc) return rc;
    if ((rc = check_append_args(c, seq, n_rows, k_new, v_new, fn))) return rc;
    std::vector<Seg> segs;
    if (seq == KVQ_ALL_SEQS) {
        for (int b = 0; b < c->batch; ++b) segs.push_back({b, b, c->len[b], 1, false});
    } else if (n_rows > 0) {
        segs.push_back({seq, 0, c->len[seq], n_rows, false});
    }
    if ((rc = launch_segments(c, k_new, v_new, segs, (hipStream_t)stream, fn))) return rc;
    for (const Seg& sg : segs) c->len[sg.seq] += sg.n;
    return KVQ_OK;
}

int kv_append_i8(kvq_cache* c, int seq, int n_rows, const float* k_new, const float* v_new, void* stream) {
    const char* fn = "kv_append_i8";
    int rc = check_cache(c, KVQ_KIND_I8, fn);
    if (rc) return rc;
    if ((rc = check_append_args(c, seq, n_rows, k_new, v_new, fn))) return rc;
    std::vector<Seg> segs;
    if (seq == KVQ_ALL_SEQS) {
        for (int b = 0; b < c->batch; ++b) segs.push_back({b, b, c->len[b], 1, false});
    } else if (n_rows > 0) {
        segs.push_back({seq, 0, c->len[seq], n_rows, false});
    }
    if ((rc = launch_segments(c, k_new, v_new, segs, (hipStream_t)stream, fn))) return rc;
    for (const Seg& sg : segs) c->len[sg.seq] += sg.n;
    return KVQ_OK;
}

int kv_append_q8(kvq_cache* c, int seq, int n_rows, const float* k_new, const float* v_new,
                 void* stream) {
    const char* fn = "kv_append_q8";
    int rc = check_cache(c, KVQ_KIND_Q8, fn);
    if (rc) return rc;
    if ((rc = check_append_args(c, seq, n_rows, k_new, v_new, fn))) return rc;
    hipStream_t s = (hipStream_t)stream;
    if (seq == KVQ_ALL_SEQS) {
        // Sequences holding >= 64 rows and not frozen freeze before the row.
        std::vector<std::pair<int, int>> fl;
        for (int b = 0; b < c->batch; ++b)
            if (!c->frozen[b] && c->len[b] >= KVQ_COL_WARMUP) fl.push_back({b, c->len[b]});
        if ((rc = launch_freeze_list(c, fl, s, fn))) return rc;
        for (auto& f : fl) c->frozen[f.first] = 1;
        std::vector<Seg> segs;
        for (int b = 0; b < c->batch; ++b) segs.push_back({b, b, c->len[b], 1, c->frozen[b] != 0});
        if ((rc = launch_segments(c, k_new, v_new, segs, s, fn))) return rc;
        for (int b = 0; b < c->batch; ++b) c->len[b] += 1;
        return KVQ_OK;
    }
    if (n_rows == 0) return KVQ_OK;
    const int L = c->len[seq];
    if (c->frozen[seq] || L + n_rows <= KVQ_COL_WARMUP) {
        std::vector<Seg> one{{seq, 0, L, n_rows, c->frozen[seq] != 0}};
        if ((rc = launch_segments(c, k_new, v_new, one, s, fn))) return rc;
        c->len[seq] = L + n_rows;
        return KVQ_OK;
    }
    // The chunk reaches a row appended while >= 64 rows are stored: rows up
    // to 64 go in unfrozen, then the freeze, then the rest against the field.
    const int n1 = std::max(0, KVQ_COL_WARMUP - L);
    if (n1 > 0) {
        std::vector<Seg> first{{seq, 0, L, n1, false}};
        if ((rc = launch_segments(c, k_new, v_new, first, s, fn))) return rc;
        c->len[seq] = L + n1;
    }
    std::vector<std::pair<int, int>> fl{{seq, c->len[seq]}};
    if ((rc = launch_freeze_list(c, fl, s, fn))) return rc;
    c->frozen[seq] = 1;
    std::vector<Seg> rest{{seq, n1, c->len[seq], n_rows - n1, true}};
    if ((rc = launch_segments(c, k_new, v_new, rest, s, fn))) return rc;
    c->len[seq] = L + n_rows;
    return KVQ_OK;
}

int kv_freeze_col_and_requant(kvq_cache* c, int seq, void* stream) {
    const char* fn = "kv_freeze_col_and_requant";
    int rc = check_cache(c, KVQ_KIND_Q8, fn);
    if (rc) return rc;
    if (seq != KVQ_ALL_SEQS && (seq < 0 || seq >= c->batch))
        return fail(KVQ_EINVAL, "%s: seq %d outside 0..%d", fn, seq, c->batch - 1);
    std::vector<std::pair<int, int>> fl;
    for (int b = 0; b < c->batch; ++b) {
        if (seq != KVQ_ALL_SEQS && b != seq) continue;
        if (!c->frozen[b] && c->len[b] > 0) fl.push_back({b, c->len[b]});
    }
    if ((rc = launch_freeze_list(c, fl, (hipStream_t)stream, fn))) return rc;
    for (auto& f : fl) c->frozen[f.first] = 1;
    return KVQ_OK;
}

size_t kvq_workspace_bytes(const kvq_cache* c, int n_q_heads) {
    if (!c || c->n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % c->n_kv_heads) return 0;
    return ws_need(c, n_q_heads / c->n_kv_heads);
}

int decode_attn_f32(const kvq_cache* c, int n_q_heads, const float* q, float* out, void* ws,
                    size_t ws_bytes, void* stream) {
    const char* fn = "decode_attn_f32";
    int rc = check_cache(c, KVQ_KIND_F32, fn);
    if (rc) return rc;
    int hpk = 0;
    if ((rc = check_decode_args(c, n_q_heads, q, out, ws, ws_bytes, fn, &hpk))) return rc;
    return run_decode(c, n_q_heads, hpk, q, out, ws, c->len, nullptr, nullptr, nullptr, nullptr,
                      (hipStream_t)stream, fn);
}

int decode_attn_q8(const kvq_cache* c, int n_q_heads, const float* q, float* out, void* ws,
                   size_t ws_bytes, void* stream) {
    const char* fn = "decode_attn_q8";
    int rc = check_cache(c, KVQ_KIND_Q8, fn);
    if (rc) return rc;
    int hpk = 0;
    if ((rc = check_decode_args(c, n_q_heads, q, out, ws, ws_bytes, fn, &hpk))) return rc;
    return run_decode(c, n_q_heads, hpk, q, out, ws, c->len, nullptr, nullptr, nullptr, nullptr,
                      (hipStream_t)stream, fn);
}

int decode_attn_q8_noalloc(const kvq_cache* c, int n_q_heads, const float* q, float* out, void* stream) {
    const char* fn = "decode_attn_q8_noalloc";
    int rc = check_cache(c, KVQ_KIND_Q8, fn);
    if (rc) return rc;
    if (n_q_heads < 1 || n_q_heads % c->n_kv_heads != 0)
        return fail(KVQ_EINVAL, "%s: n_q_heads %d is not a multiple of n_kv_heads %d", fn, n_q_heads, c->n_kv_heads);
    const int hpk = n_q_heads / c->n_kv_heads;
    if (hpk != 1 && hpk != 2 && hpk != 4 && hpk != 8)
        return fail(KVQ_EINVAL, "%s: group size %d not in {1,2,4,8}", fn, hpk);
    if (!q || !out) return fail(KVQ_EINVAL, "%s: null q/out", fn);
    if (!aligned16(q) || !aligned16(out)) return fail(KVQ_EINVAL, "%s: q/out not 16-byte aligned", fn);
    const size_t need = ws_need(c, hpk);
    if (need > kScratchBytes)
        return fail(KVQ_EINVAL, "%s: this cache needs %zu bytes of workspace, more than the %zu of the static one "
                    "(use decode_attn_q8 with a workspace)", fn, need, kScratchBytes);
    // the device array replaces the caller's workspace; nothing in it needs
    // clearing (the decode kernel writes every partial the combine reads)
    void* ws = scratch_address();
    if (!ws) return fail(KVQ_EDEVICE, "%s: no device address for the static workspace", fn);
    return run_decode(c, n_q_heads, hpk, q, out, ws, c->len, nullptr, nullptr, nullptr, nullptr,
                      (hipStream_t)stream, fn);
}

int decode_attn_i8(const kvq_cache* c, int n_q_heads, const float* q, float* out, void* ws, size_t ws_bytes,
                   void* stream) {
    const char* fn = "decode_attn_i8";
    int rc = check_cache(c, KVQ_KIND_I8, fn);
    if (rc) return rc;
    int hpk = 0;
    if ((rc = check_decode_args(c, n_q_heads, q, out, ws, ws_bytes, fn, &hpk))) return rc;
    return run_decode(c, n_q_heads, hpk, q, out, ws, c->len, nullptr, nullptr, nullptr, nullptr,
                      (hipStream_t)stream, fn);
}

int decode_attn_f32_ex(const kvq_cache* c, int n_q_heads, const float* q, float* out,
                       const kvq_decode_opts* opts, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "decode_attn_f32_ex";
    int rc = check_cache(c, KVQ_KIND_F32, fn);
    if (rc) return rc;
    int hpk = 0;
    if ((rc = check_decode_args(c, n_q_heads, q, out, ws, ws_bytes, fn, &hpk))) return rc;
    if ((rc = check_decode_opts(c, opts, fn))) return rc;
    return run_decode(c, n_q_heads, hpk, q, out, ws, c->len, nullptr, nullptr, nullptr, opts,
                      (hipStream_t)stream, fn);
}

int decode_attn_q8_ex(const kvq_cache* c, int n_q_heads, const float* q, float* out,
                      const kvq_decode_opts* opts, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "decode_attn_q8_ex";
    int rc = check_cache(c, KVQ_KIND_Q8, fn);
    if (rc) return rc;
    int hpk = 0;
    if ((rc = check_decode_args(c, n_q_heads, q, out, ws, ws_bytes, fn, &hpk))) return rc;
    if ((rc = check_decode_opts(c, opts, fn))) return rc;
    return run_decode(c, n_q_heads, hpk, q, out, ws, c->len, nullptr, nullptr, nullptr, opts,
                      (hipStream_t)stream, fn);
}

int rswa_record_prefill(kvq_cache* c, kvq_ring* rings, int seq) {
    const char* fn = "rswa_record_prefill";
    int rc = check_ring_cache(c, fn);
    if (rc) return rc;
    if (!rings) return fail(KVQ_EINVAL, "%s: null rings", fn);
    if (seq < 0 || seq >= c->batch) return fail(KVQ_EINVAL, "%s: seq %d outside 0..%d", fn, seq, c->batch - 1);
    if ((int64_t)c->len[seq] + KVQ_RING_WINDOW > c->capacity)
        return fail(KVQ_ECAPACITY, "%s: prefill %d + ring %d exceeds capacity %d", fn, c->len[seq],
                    KVQ_RING_WINDOW, c->capacity);
    // a new prefill starts a new lineage ([P3] record_prefill)
    if (rings[seq].epoch == INT32_MAX) return fail(KVQ_ESTATE, "%s: lineage epoch exhausted", fn);
    rings[seq].prefill_len = c->len[seq];
    rings[seq].ring_len = 0;
    rings[seq].ring_pos = 0;
    rings[seq].epoch += 1;
    rings[seq].writes = 0;
    return KVQ_OK;
}


int rswa_checkpoint(const kvq_cache* c, const kvq_ring* rings, int seq, kvq_ring_checkpoint* cp) {
    const char* fn = "rswa_checkpoint";
    int rc = check_ring_cache(c, fn);
    if (rc) return rc;
    if (!rings || !cp) return fail(KVQ_EINVAL, "%s: null rings/checkpoint", fn);
    if (seq < 0 || seq >= c->batch) return fail(KVQ_EINVAL, "%s: seq %d outside 0..%d", fn, seq, c->batch - 1);
    take_checkpoint(c, rings[seq], seq, -1, cp);
    return KVQ_OK;
}

int rswa_rollback_to(kvq_cache* c, kvq_ring* rings, int seq, const kvq_ring_checkpoint* cp) {
    const char* fn = "rswa_rollback_to";
    int rc = check_ring_cache(c, fn);
    if (rc) return rc;
    if (!rings || !cp) return fail(KVQ_EINVAL, "%s: null rings/checkpoint", fn);
    if (seq < 0 || seq >= c->batch) return fail(KVQ_EINVAL, "%s: seq %d outside 0..%d", fn, seq, c->batch - 1);
    if (cp->cache != c || cp->seq != seq || cp->stream != -1)
        return fail(KVQ_ESTATE, "%s: checkpoint belongs to another cache, sequence or a shared stream", fn);
    kvq_ring& r = rings[seq];
    if ((rc = rollback_ring(r, cp, fn))) return rc;
    c->len[seq] = r.prefill_len + r.ring_len;
    return KVQ_OK;
}

int rswa_shared_checkpoint(const kvq_cache* c, int seq, const kvq_ring* rings, int n_streams, int s,
                           kvq_ring_checkpoint* cp) {
    const char* fn = "rswa_shared_checkpoint";
    if (!cp) return fail(KVQ_EINVAL, "%s: null checkpoint", fn);
    const int rc = check_shared_stream(c, seq, rings, n_streams, s, fn);
    if (rc) return rc;
    take_checkpoint(c, rings[s], seq, s, cp);
    return KVQ_OK;
}

int rswa_shared_rollback_to(kvq_cache* c, int seq, kvq_ring* rings, int n_streams, int s,
                            const kvq_ring_checkpoint* cp) {
    const char* fn = "rswa_shared_rollback_to";
    if (!cp) return fail(KVQ_EINVAL, "%s: null checkpoint", fn);
    const int rc = check_shared_stream(c, seq, rings, n_streams, s, fn);
    if (rc) return rc;
    if (cp->cache != c || cp->seq != seq || cp->stream != s)
        return fail(KVQ_ESTATE, "%s: checkpoint belongs to another cache, sequence or stream", fn);
    // the rings' rows stay reserved: len[seq] does not move
    return rollback_ring(rings[s], cp, fn);
}

int kv_truncate_last(kvq_cache* c, int seq, int n_drop) {
    const char* fn = "kv_truncate_last";
    int rc = check_cache(c, 0, fn);
    if (rc) return rc;
    if (n_drop < 0) return fail(KVQ_EINVAL, "%s: n_drop %d < 0", fn, n_drop);
    if (seq != KVQ_ALL_SEQS && (seq < 0 || seq >= c->batch))
        return fail(KVQ_EINVAL, "%s: seq %d outside 0..%d", fn, seq, c->batch - 1);
    const int b0 = seq == KVQ_ALL_SEQS ? 0 : seq, b1 = seq == KVQ_ALL_SEQS ? c->batch : seq + 1;
    for (int b = b0; b < b1; ++b) c->len[b] -= std::min(n_drop, c->len[b]);
    return KVQ_OK;
}

int kv_trim_window(kvq_cache* c, int seq, int64_t* base, int w, int slack, int align, int64_t anchor,
                   int* dropped, void* stream) {
    const char* fn = "kv_trim_window";
    int rc = check_cache(c, 0, fn);
    if (rc) return rc;
    if (!base) return fail(KVQ_EINVAL, "%s: null base", fn);
    if (seq != KVQ_ALL_SEQS && (seq < 0 || seq >= c->batch))
        return fail(KVQ_EINVAL, "%s: seq %d outside 0..%d", fn, seq, c->batch - 1);
    const int b0 = seq == KVQ_ALL_SEQS ? 0 : seq, b1 = seq == KVQ_ALL_SEQS ? c->batch : seq + 1;
    // base / dropped: one entry, or one per sequence for KVQ_ALL_SEQS
    int64_t* bases = seq == KVQ_ALL_SEQS ? base : base - b0;
    int* drops = !dropped ? nullptr : seq == KVQ_ALL_SEQS ? dropped : dropped - b0;
    if (w < 0 || slack < 0 || align < 0)
        return fail(KVQ_EINVAL, "%s: w %d, slack %d, align %d must be >= 0", fn, w, slack, align);
    for (int b = b0; b < b1; ++b)
        if (bases[b] < 0) return fail(KVQ_EINVAL, "%s: base[%d] = %lld must be >= 0", fn, b, (long long)bases[b]);
    // [P2] trim_window_anchored, step by step, for each sequence
    std::vector<TrimMove> moves;
    std::vector<int64_t> new_base(b1 - b0);
    for (int b = b0; b < b1; ++b) {
        new_base[b - b0] = bases[b];
        const int64_t n = c->len[b];
        if (w == 0 || n <= 2 * (int64_t)w) continue;
        if (c->kind == KVQ_KIND_Q8 && !c->frozen[b]) continue;
        const int64_t al = std::max(align, 1);
        int64_t keep_from = std::max<int64_t>(bases[b] + n - (w + slack), 0);
        if (anchor >= 0) keep_from = std::min(keep_from, std::max<int64_t>(anchor - (w + slack), 0));
        const int64_t nb = keep_from / al * al;
        if (nb <= bases[b]) continue;
        const int d = (int)(nb - bases[b]);            // < n: nb <= keep_from < base + n
        moves.push_back({b, d, (int)(n - d)});
        new_base[b - b0] = nb;
    }
    if (c->n_live > 0 && !moves.empty()) {
        MoveArgs m;
        memset(&m, 0, sizeof m);
        m.k = c->k;
        m.v = c->v;
        m.kq = c->kq;
        m.ks = c->ks;
        m.vq = c->vq;
        m.vs = c->vs;
        m.n_live = c->n_live;
        m.capacity = c->capacity;
        m.kind = c->kind;
        if ((rc = device_status(launch_trim_moves(m, moves.data(), (int)moves.size(), (hipStream_t)stream), fn)))
            return rc;
    }
    for (int b = b0; b < b1; ++b) {
        const int d = (int)(new_base[b - b0] - bases[b]);
        c->len[b] -= d;
        bases[b] = new_base[b - b0];
        if (drops) drops[b] = d;
    }
    return KVQ_OK;
}

int rswa_decode(kvq_cache* c, kvq_ring* rings, int n_q_heads, const float* q, const float* k_new,
                const float* v_new, float* out, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "rswa_decode";
    int rc = check_ring_cache(c, fn);
    if (rc) return rc;
    int hpk = 0;
    if ((rc = check_decode_args(c, n_q_heads, q, out, ws, ws_bytes, fn, &hpk))) return rc;
    if (!rings) return fail(KVQ_EINVAL, "%s: null rings", fn);
    if (!k_new || !v_new) return fail(KVQ_EINVAL, "%s: null k_new/v_new", fn);
    if (!aligned16(k_new) || !aligned16(v_new)) return fail(KVQ_EINVAL, "%s: k_new/v_new not 16-byte aligned", fn);
    std::vector<int32_t> lens(c->batch), wrows(c->batch);
    std::vector<kvq_ring> next(rings, rings + c->batch);
    for (int b = 0; b < c->batch; ++b) {
        kvq_ring& r = next[b];
        if (r.prefill_len < 0) return fail(KVQ_ESTATE, "%s: sequence %d: decode before record_prefill", fn, b);
        if ((int64_t)r.prefill_len + KVQ_RING_WINDOW > c->capacity)
            return fail(KVQ_ECAPACITY, "%s: sequence %d: prefill %d + ring exceeds capacity %d", fn, b,
                        r.prefill_len, c->capacity);
        if (r.ring_len < 0 || r.ring_len > KVQ_RING_WINDOW || r.ring_pos < 0 || r.ring_pos >= KVQ_RING_WINDOW)
            return fail(KVQ_ESTATE, "%s: sequence %d: corrupt ring cursors", fn, b);
        if (c->len[b] != r.prefill_len + r.ring_len)
            return fail(KVQ_ESTATE, "%s: sequence %d: len %d != prefill %d + ring %d (appended since record?)", fn,
                        b, c->len[b], r.prefill_len, r.ring_len);
        int slot;
        if (r.ring_len < KVQ_RING_WINDOW) {   // ring not full yet: next free slot, nothing evicted
            slot = r.ring_len;
            r.ring_len += 1;
            r.ring_pos = r.ring_len % KVQ_RING_WINDOW;
        } else {                              // steady state: overwrite in place
            slot = r.ring_pos;
            r.ring_pos = (r.ring_pos + 1) % KVQ_RING_WINDOW;
        }
        r.writes += 1;
        wrows[b] = r.prefill_len + slot;
        lens[b] = r.prefill_len + r.ring_len;
    }
    // the ring row is written inside the decode kernel, by the wave whose
    // share holds it (on the i8 kind quantised there with quantize_row_i8)
    if ((rc = run_decode(c, n_q_heads, hpk, q, out, ws, lens.data(), wrows.data(), k_new, v_new, nullptr,
                         (hipStream_t)stream, fn)))
        return rc;
    for (int b = 0; b < c->batch; ++b) {
        rings[b] = next[b];
        c->len[b] = lens[b];
    }
    return KVQ_OK;
}

size_t kvq_verify_workspace_bytes(const kvq_cache* c, int n_q_heads, int n_draft) {
    if (!c || c->n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % c->n_kv_heads || n_draft < 1) return 0;
    const int nq = n_draft * (n_q_heads / c->n_kv_heads);
    if (nq > kVerifyMaxQ) return 0;
    return ws_need(c, nq);
}

int rswa_verify(const kvq_cache* c, const kvq_ring* rings, int n_q_heads, int n_draft, const float* q,
                const float* k_draft, const float* v_draft, float* out, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "rswa_verify";
    int rc = check_ring_cache(c, fn);
    if (rc) return rc;
    if (n_q_heads < 1 || n_q_heads % c->n_kv_heads != 0)
        return fail(KVQ_EINVAL, "%s: n_q_heads %d is not a multiple of n_kv_heads %d", fn, n_q_heads, c->n_kv_heads);
    const int hpk = n_q_heads / c->n_kv_heads;
    if (n_draft < 1 || n_draft * hpk > kVerifyMaxQ)
        return fail(KVQ_EINVAL, "%s: n_draft %d x group %d must be within 1..%d", fn, n_draft, hpk, kVerifyMaxQ);
    if (!rings || !q || !k_draft || !v_draft || !out || !ws) return fail(KVQ_EINVAL, "%s: null argument", fn);
    if (!aligned16(q) || !aligned16(k_draft) || !aligned16(v_draft) || !aligned16(out) || !aligned16(ws))
        return fail(KVQ_EINVAL, "%s: q/k_draft/v_draft/out/workspace not 16-byte aligned", fn);
    const bool i8 = c->kind == KVQ_KIND_I8;
    const size_t need = ws_need(c, n_draft * hpk);
    if (ws_bytes < need) return fail(KVQ_EINVAL, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    for (int b = 0; b < c->batch; ++b) {
        const kvq_ring& r = rings[b];
        if (r.prefill_len < 0) return fail(KVQ_ESTATE, "%s: sequence %d: verify before record_prefill", fn, b);
        if (r.ring_len < 0 || r.ring_len > KVQ_RING_WINDOW || r.ring_pos < 0 || r.ring_pos >= KVQ_RING_WINDOW)
            return fail(KVQ_ESTATE, "%s: sequence %d: corrupt ring cursors", fn, b);
        if (c->len[b] != r.prefill_len + r.ring_len)
            return fail(KVQ_ESTATE, "%s: sequence %d: len %d != prefill %d + ring %d", fn, b, c->len[b], r.prefill_len,
                        r.ring_len);
    }
    VerifyArgs a;
    memset(&a, 0, sizeof a);
    a.q = q;
    a.out = out;
    a.k = c->k;
    a.v = c->v;
    a.kd = k_draft;
    a.vd = v_draft;
    a.ws_acc = (float*)ws;
    a.ws_ml = (float*)ws + ws_slots(c) * (size_t)(n_draft * hpk) * kHD;
    a.n_kv_heads = c->n_kv_heads;
    a.n_live = c->n_live;
    a.n_q_heads = n_q_heads;
    a.hpk = hpk;
    a.capacity = c->capacity;
    a.n_draft = n_draft;
    a.nq = n_draft * hpk;
    fill_live(c, a.live_head);
    memcpy(a.live_slot, c->live_slot, sizeof a.live_slot);
    if (i8) {
        // [P3] write_decode_step of the drafts on a clone of the int8 mirror:
        // the kernel quantises each draft row where it reads it (nothing is
        // written to the cache)
        a.kq = c->kq;
        a.ks = c->ks;
        a.vq = c->vq;
        a.vs = c->vs;
    }
    for (int s0 = 0; s0 < c->batch; s0 += kSeqPerLaunch) {
        const int ns = std::min(kSeqPerLaunch, c->batch - s0);
        a.seq0 = s0;
        a.n_seq = ns;
        int64_t tiles = 0;
        for (int j = 0; j < ns; ++j) {
            const kvq_ring& r = rings[s0 + j];
            a.prefill[j] = r.prefill_len;
            a.ring_len[j] = r.ring_len;
            a.ring_oldest[j] = r.ring_len < KVQ_RING_WINDOW ? 0 : r.ring_pos;
            a.len[j] = r.prefill_len + r.ring_len + n_draft;
            a.ntile[j] = (a.len[j] + kTileRows - 1) / kTileRows;
            a.tile_base[j] = (int32_t)tiles;
            tiles += (int64_t)a.ntile[j] * c->n_live;
            if (tiles >= ((int64_t)1 << 31)) return fail(KVQ_EINVAL, "%s: more than 2^31 tiles in one launch", fn);
        }
        a.tile_base[ns] = (int32_t)tiles;
        a.n_tiles = (int)tiles;
        if ((rc = device_status(i8 ? launch_verify_i8(a, (hipStream_t)stream) : launch_verify_f32(a, (hipStream_t)stream),
                                fn)))
            return rc;
    }
    return KVQ_OK;
}

int rswa_shared_record_prefill(kvq_cache* c, int seq, kvq_ring* rings, int n_streams) {
    const char* fn = "rswa_shared_record_prefill";
    int rc = check_ring_cache(c, fn);
    if (rc) return rc;
    if (!rings) return fail(KVQ_EINVAL, "%s: null rings", fn);
    if (seq < 0 || seq >= c->batch) return fail(KVQ_EINVAL, "%s: seq %d outside 0..%d", fn, seq, c->batch - 1);
    if (n_streams < 1 || n_streams > kVerifyMaxQ)
        return fail(KVQ_EINVAL, "%s: n_streams %d outside 1..%d", fn, n_streams, kVerifyMaxQ);
    const int pre = c->len[seq];
    if ((int64_t)pre + (int64_t)KVQ_RING_WINDOW * n_streams > c->capacity)
        return fail(KVQ_ECAPACITY, "%s: prefill %d + %d rings of %d exceeds capacity %d", fn, pre, n_streams,
                    KVQ_RING_WINDOW, c->capacity);
    for (int s = 0; s < n_streams; ++s)
        if (rings[s].epoch == INT32_MAX) return fail(KVQ_ESTATE, "%s: stream %d: lineage epoch exhausted", fn, s);
    for (int s = 0; s < n_streams; ++s) {
        rings[s].prefill_len = pre;
        rings[s].ring_len = 0;
        rings[s].ring_pos = 0;
        rings[s].epoch += 1;
        rings[s].writes = 0;
    }
    c->len[seq] = pre + KVQ_RING_WINDOW * n_streams;       // the rings' rows are reserved
    return KVQ_OK;
}

int rswa_shared_decode(kvq_cache* c, int seq, kvq_ring* rings, int n_streams, int n_q_heads, const float* q,
                       const float* k_new, const float* v_new, float* out, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "rswa_shared_decode";
    int rc = check_ring_cache(c, fn);
    if (rc) return rc;
    if (seq < 0 || seq >= c->batch) return fail(KVQ_EINVAL, "%s: seq %d outside 0..%d", fn, seq, c->batch - 1);
    if (n_q_heads < 1 || n_q_heads % c->n_kv_heads != 0)
        return fail(KVQ_EINVAL, "%s: n_q_heads %d is not a multiple of n_kv_heads %d", fn, n_q_heads, c->n_kv_heads);
    const int hpk = n_q_heads / c->n_kv_heads;
    if (n_streams < 1 || n_streams * hpk > kVerifyMaxQ)
        return fail(KVQ_EINVAL, "%s: n_streams %d x group %d must be within 1..%d", fn, n_streams, hpk, kVerifyMaxQ);
    if (!rings || !q || !k_new || !v_new || !out || !ws) return fail(KVQ_EINVAL, "%s: null argument", fn);
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out) || !aligned16(ws))
        return fail(KVQ_EINVAL, "%s: q/k_new/v_new/out/workspace not 16-byte aligned", fn);
    const size_t need = ws_need(c, n_streams * hpk);
    if (ws_bytes < need) return fail(KVQ_EINVAL, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    const int pre = rings[0].prefill_len;
    if (pre < 0) return fail(KVQ_ESTATE, "%s: decode before rswa_shared_record_prefill", fn);
    if ((int64_t)c->len[seq] != (int64_t)pre + (int64_t)KVQ_RING_WINDOW * n_streams)
        return fail(KVQ_ESTATE, "%s: len %d != prefill %d + %d rings (another group size, or appended since)", fn,
                    c->len[seq], pre, n_streams);
    std::vector<kvq_ring> next(rings, rings + n_streams);
    VerifyArgs a;
    memset(&a, 0, sizeof a);
    for (int s = 0; s < n_streams; ++s) {
        kvq_ring& r = next[s];
        if (r.prefill_len != pre) return fail(KVQ_ESTATE, "%s: stream %d: prefill %d != %d", fn, s, r.prefill_len, pre);
        if (r.ring_len < 0 || r.ring_len > KVQ_RING_WINDOW || r.ring_pos < 0 || r.ring_pos >= KVQ_RING_WINDOW)
            return fail(KVQ_ESTATE, "%s: stream %d: corrupt ring cursors", fn, s);
        a.sring[s] = r.ring_len;                  // slots live before the step
        int slot;                                 // [P3] write_decode_step, as rswa_decode
        if (r.ring_len < KVQ_RING_WINDOW) {
            slot = r.ring_len;
            r.ring_len += 1;
            r.ring_pos = r.ring_len % KVQ_RING_WINDOW;
        } else {
            slot = r.ring_pos;
            r.ring_pos = (r.ring_pos + 1) % KVQ_RING_WINDOW;
        }
        r.writes += 1;
        a.swrow[s] = pre + KVQ_RING_WINDOW * s + slot;
    }
    const bool i8 = c->kind == KVQ_KIND_I8;
    if (i8) {
        // the int8 mirror: the kernel quantises each step row where it reads
        // it and stores its codes in the stream's ring slot
        a.kq = c->kq;
        a.ks = c->ks;
        a.vq = c->vq;
        a.vs = c->vs;
    }
    a.shared = 1;
    a.q = q;
    a.out = out;
    a.k = c->k;
    a.v = c->v;
    a.k_store = c->k;
    a.v_store = c->v;
    a.kd = k_new;
    a.vd = v_new;
    a.ws_acc = (float*)ws;
    a.ws_ml = (float*)ws + ws_slots(c) * (size_t)(n_streams * hpk) * kHD;
    a.n_kv_heads = c->n_kv_heads;
    a.n_live = c->n_live;
    a.n_q_heads = n_q_heads;
    a.hpk = hpk;
    a.capacity = c->capacity;
    a.n_draft = n_streams;
    a.nq = n_streams * hpk;
    fill_live(c, a.live_head);
    memcpy(a.live_slot, c->live_slot, sizeof a.live_slot);
    a.seq0 = seq;
    a.n_seq = 1;
    a.prefill[0] = pre;
    a.len[0] = c->len[seq] + n_streams;                     // reference, rings, then the step rows
    a.ntile[0] = (a.len[0] + kTileRows - 1) / kTileRows;
    a.tile_base[0] = 0;
    a.tile_base[1] = a.ntile[0] * c->n_live;
    a.n_tiles = a.tile_base[1];
    if ((rc = device_status(i8 ? launch_verify_i8(a, (hipStream_t)stream) : launch_verify_f32(a, (hipStream_t)stream),
                            fn)))
        return rc;
    for (int s = 0; s < n_streams; ++s) rings[s] = next[s];
    return KVQ_OK;
}

const char* kvq_last_error(void) { return g_err.c_str(); }

}  // extern "C"
