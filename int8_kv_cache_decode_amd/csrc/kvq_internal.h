// kvq_internal.h -- argument blocks and launchers shared by the library's
// host code (kvq_api.hip) and its kernels (kvq_codec.hip, kvq_decode.hip).
//
// Per-sequence values (lengths, destination rows, ring rows, work offsets)
// travel inside the kernel-argument block, so a call never has to stage a
// table in device memory.  One launch covers at most kSeqPerLaunch
// sequences; larger batches are processed in consecutive launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kHD = KVQ_HEAD_DIM;           // channels per head
constexpr int kKGroup = KVQ_K_GROUP;        // K channels per scale
constexpr int kKScales = kHD / kKGroup;     // K scales per row (4)
constexpr int kSeqPerLaunch = 128;

// Work split of the decode kernels (stream-K): the rows of every (sequence,
// live KV head) of a launch are cut into 16-row tiles, laid end to end in
// sequence-major, head-minor order, and the tile stream is divided into
// n_shares contiguous, equal shares, one per wave of a grid that is resident
// all at once.  A wave folds its share segment by segment and writes one
// partial per segment its share touches, in slot share + segment; the
// combine kernel merges the slots of a segment, a contiguous range.
// kMaxWaves bounds n_shares (and so the workspace): 256 compute units x 32
// wave slots.
constexpr int kTileRows = 16;
constexpr int kMaxWaves = 8192;

// K codes of the int8 kinds are stored tile-major, in the order the matrix
// cores read them: the rows of a (sequence, live head) form 16-row tiles of
// 2 KB, and within a tile the 16-byte piece (row n, channels 16 c .. 16 c +
// 15) sits at (c / 4) * 1024 + (c % 4) * 256 + n * 16.  One MFMA operand
// load of a tile (64 lanes x 16 bytes: lane 16 (c % 4) + n) is then 1 KB of
// whole lines.  A (sequence, live head) holds kq_rows(capacity) rows: the
// capacity rounded up to whole tiles.  The other buffers stay row-major.
__host__ __device__ inline int kq_rows(int capacity) { return (capacity + kTileRows - 1) & ~(kTileRows - 1); }
__host__ __device__ inline uint32_t kq_offset(int row, int ch) {
    return (uint32_t)(row >> 4) * 2048u + (uint32_t)(ch >> 6) * 1024u + (uint32_t)((ch >> 4) & 3) * 256u +
           (uint32_t)(row & 15) * 16u + (uint32_t)(ch & 15);
}

// ---- codec ---------------------------------------------------------------
struct AppendArgs {
    const float* k_new;        // source rows [src_row][n_kv_heads][128]
    const float* v_new;
    float* k;                  // f32 cache storage
    float* v;
    int8_t* kq;                // q8 cache storage
    float* ks;
    int8_t* vq;
    float* vs;
    const float* kcol;
    const float* vcol;
    int n_kv_heads;
    int n_live;
    int capacity;
    int n_seq;                 // sequences in this launch
    int8_t live_head[KVQ_MAX_KV_HEADS];      // KV head of live slot
    int32_t seq[kSeqPerLaunch];              // absolute sequence index
    int32_t src_row0[kSeqPerLaunch];         // first source row of the sequence
    int32_t dst_row0[kSeqPerLaunch];         // first destination row
    int32_t frozen[kSeqPerLaunch];           // q8: quantise against the column field
};

struct FreezeArgs {
    int8_t* kq;
    float* ks;
    int8_t* vq;
    float* vs;
    float* kcol;
    float* vcol;
    int n_live;
    int capacity;
    int n_seq;
    int32_t seq[kSeqPerLaunch];
    int32_t n[kSeqPerLaunch];                // rows to freeze over
};

// Front-trim moves ([P2] trim_window): sequence seq[i] drops its first d[i]
// rows, rows [d, d + keep) of every live head going to rows [0, keep) in
// order.  The moves run in rounds of at most d rows per sequence, one launch
// per round for all the sequences that still have rows to move, so that a
// launch's source and destination rows never overlap.
struct MoveArgs {
    float* k;
    float* v;
    int8_t* kq;
    float* ks;
    int8_t* vq;
    float* vs;
    int n_live;
    int capacity;
    int kind;       // KVQ_KIND_*: which buffers move
    int n_seq;      // sequences in this launch
    int32_t seq[kSeqPerLaunch];
    int32_t src[kSeqPerLaunch];   // first source row of the round's chunk
    int32_t dst[kSeqPerLaunch];   // first destination row
    int32_t m[kSeqPerLaunch];     // rows the round moves
};
struct TrimMove {
    int seq, d, keep;
};

// grid (n_rows, n_seq, n_live)
hipError_t launch_append_f32(const AppendArgs& a, int n_rows, hipStream_t s);
hipError_t launch_append_q8(const AppendArgs& a, int n_rows, hipStream_t s);
hipError_t launch_append_i8(const AppendArgs& a, int n_rows, hipStream_t s);
// grid (n_live, n_seq)
hipError_t launch_freeze(const FreezeArgs& a, hipStream_t s);
// the moves of every listed sequence, one launch per round (a: buffers and
// geometry; its per-sequence fields are filled here)
hipError_t launch_trim_moves(const MoveArgs& a, const TrimMove* moves, int count, hipStream_t s);

// ---- decode --------------------------------------------------------------
struct DecodeArgs {
    const float* q;            // [batch][n_q_heads][128]
    float* out;                // [batch][n_q_heads][128]
    const float* k;            // f32 storage
    const float* v;
    const int8_t* kq;          // q8 storage
    const float* ks;
    const int8_t* vq;
    const float* vs;
    const float* kcol;
    const float* vcol;
    float* ws_acc;             // [slots][hpk][128] partial weighted V sums
    float* ws_ml;              // [slots][hpk][2]   partial (max, sum) in log2 units
    const float* k_new;        // R-SWA step K/V [batch][n_kv_heads][128] (or null)
    const float* v_new;
    float* k_store;            // writable f32 storage for the ring write
    float* v_store;
    int8_t* kq_store;          // writable int8 storage for the ring write (per-row int8 kind)
    float* ks_store;
    int8_t* vq_store;
    float* vs_store;
    int n_kv_heads;
    int n_live;
    int n_q_heads;
    int hpk;
    int capacity;
    int n_seq;                 // sequences in this launch
    int seq0;                  // first absolute sequence of this launch
    int n_tiles;               // 16-row tiles of the launch over all (sequence, live head)
    int n_shares;              // shares of the tile stream (set by the launcher, <= n_tiles)
    double softcap2;           // logit soft-cap in log2 units (softcap * log2 e), 0 = off
    const float* sinks;        // [n_q_heads] learned sink logits (natural units), or null
    int8_t live_head[KVQ_MAX_KV_HEADS];      // KV head of live slot
    int8_t live_slot[KVQ_MAX_KV_HEADS];      // live slot of KV head, -1 dead
    int32_t tile_base[kSeqPerLaunch + 1];    // first tile of each sequence (its live heads in order)
    int32_t ntile[kSeqPerLaunch];            // tiles per (sequence, live head) = ceil((len - start) / 16)
    int32_t first[kSeqPerLaunch];            // first visible row (rows [first, len) are attended)
    int32_t start[kSeqPerLaunch];            // first row of the tile stream: first, rounded down to
                                             // a multiple of 16 for the int8 kinds (whole K tiles)
    int32_t len[kSeqPerLaunch];              // rows stored
    int32_t wrow[kSeqPerLaunch];             // R-SWA row taken from k_new/v_new, -1 none
    uint8_t frozen[kSeqPerLaunch];           // q8: column fields hold the frozen RMS
};

// A byte of a kernel-argument array, read through its aligned dword: with a
// wave-uniform index that is one scalar load (the byte itself would take a
// vector load and a wait for it, a microsecond at a piece's start).
template <class T>
__device__ __forceinline__ int arg_byte(const T* arr, int i) {
    static_assert(sizeof(T) == 1, "a byte array");
    const int32_t w = reinterpret_cast<const int32_t*>(arr)[i >> 2];
    return (int)(T)(w >> (8 * (i & 3)));
}

// Partial slots a launch can use: n_shares + n_seq * n_live.
inline size_t max_slots(int n_seq, int n_live) { return (size_t)kMaxWaves + (size_t)n_seq * n_live; }

// K-token R-SWA verify ([P3] verify_attention): per sequence, the segment
// of a live head is its cache rows [0, prefill + ring_len) followed by the
// n_draft draft rows, read from kd/vd.
struct VerifyArgs {
    const float* q;            // [batch][n_draft][n_q_heads][128]
    float* out;                // [batch][n_draft][n_q_heads][128]
    const float* k;            // f32 storage
    const float* v;
    const float* kd;           // draft K/V [batch][n_draft][n_kv_heads][128]
    const float* vd;
    float* ws_acc;             // [slots][nq][128]
    float* ws_ml;              // [slots][nq][2]
    int n_kv_heads;
    int n_live;
    int n_q_heads;
    int hpk;
    int capacity;
    int n_seq;
    int seq0;
    int n_tiles;
    int n_shares;
    int n_draft;
    int nq;                    // n_draft * hpk queries per KV head (<= 16)
    int8_t live_head[KVQ_MAX_KV_HEADS];
    int8_t live_slot[KVQ_MAX_KV_HEADS];
    int32_t tile_base[kSeqPerLaunch + 1];
    int32_t ntile[kSeqPerLaunch];
    int32_t len[kSeqPerLaunch];              // prefill + ring_len + n_draft
    int32_t prefill[kSeqPerLaunch];
    int32_t ring_len[kSeqPerLaunch];
    int32_t ring_oldest[kSeqPerLaunch];      // slot of the oldest live ring token
    // Shared-reference decode (one launch per shared group: n_seq = 1; the
    // n_draft "drafts" are the streams, kd / vd their step rows, q / out are
    // [n_draft][n_q_heads][128]; len = prefill + 128 n_draft + n_draft).
    // Stream s's ring is rows prefill + 128 s ..
    int shared;
    float* k_store;                          // writable f32 storage for the ring writes
    float* v_store;
    int32_t sring[16];                       // ring slots of stream s live before its step
    int32_t swrow[16];                       // row of the sequence that stream s's step writes
    // per-row int8 kind: the cache's codes and row scales (the drafts and step
    // rows are quantised inside the kernel), writable for the ring writes
    int8_t* kq;
    float* ks;
    int8_t* vq;
    float* vs;
};
constexpr int kVerifyMaxQ = 16;

// the byte arrays read with arg_byte start on a dword and hold whole dwords
static_assert(offsetof(AppendArgs, live_head) % 4 == 0, "");
static_assert(offsetof(DecodeArgs, live_head) % 4 == 0 && offsetof(DecodeArgs, live_slot) % 4 == 0 &&
              offsetof(DecodeArgs, frozen) % 4 == 0, "");
static_assert(offsetof(VerifyArgs, live_head) % 4 == 0 && offsetof(VerifyArgs, live_slot) % 4 == 0, "");
static_assert(KVQ_MAX_KV_HEADS % 4 == 0 && kSeqPerLaunch % 4 == 0, "");

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s);
hipError_t launch_verify_f32(const VerifyArgs& a, hipStream_t s);   // a.shared: the shared-reference decode
hipError_t launch_verify_i8(const VerifyArgs& a, hipStream_t s);    // the same on the per-row int8 kind
hipError_t launch_decode_q8(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_i8(const DecodeArgs& a, hipStream_t s);

}  // namespace kvq
