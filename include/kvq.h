/*
 * kvq.h -- C ABI of the MI355X (gfx950) decode-attention library over a
 * head-major KV cache: f32, int8 with column fields ("q8_2f", [P1]/[P2]),
 * or per-row int8 ([P3]'s int8 mirror).
 *
 * Sources (web pages the operations come from):
 *   [P1] cortiq-engine 0.3.4, src/cortiq_engine/kv_cache.rs
 *        (LayerKvCache: head-major storage, quant_row, freeze_cols, append,
 *         attend, attend_group)
 *   [P2] cortiq-engine 0.8.49, src/cortiq_engine/kv_cache.rs (same codec)
 *   [P3] franken_ocr 0.8.0, src/native_engine/rswa.rs
 *        (RingCache: record_prefill, write_decode_step, decode_attention,
 *         fold, attention, batched_decode_attention)
 *
 * Conventions for every call below
 *   - Status: 0 (KVQ_OK) on success, a negative KVQ_E* code otherwise; the
 *     message of the last failure on the calling thread is returned by
 *     kvq_last_error().
 *   - All validation happens on the host BEFORE anything is enqueued: a call
 *     that fails leaves the cache (device buffers and host counters) exactly
 *     as it was.  The one exception is KVQ_EDEVICE (a launch the HIP runtime
 *     refused), which is reported after the fact.
 *   - Ownership: the caller allocates and owns every buffer -- the kvq_cache
 *     and kvq_ring structs, the host counter arrays they point to, and every
 *     device buffer (cache storage, q, k_new/v_new, out, workspace).  The
 *     library never allocates, frees or synchronises.
 *   - Device pointers are HIP device addresses on the current device.  Calls
 *     are asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *     Host counters (len, frozen, ring cursors) are updated when the work is
 *     enqueued, i.e. they describe the cache as it will be once the stream
 *     reaches that point.
 *   - Calls that share a cache, or a workspace, must be ordered (same stream
 *     or explicit synchronisation); overlapping calls race.
 *   - Only head_dim == 128 is accepted.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_HEAD_DIM      128   /* channels per head (the only supported value) */
#define KVQ_K_GROUP       32    /* K channels per scale ([P1] const KV_K_GROUP) */
#define KVQ_COL_WARMUP    64    /* rows before the column field freezes ([P1] const KV_COL_WARMUP) */
#define KVQ_RING_WINDOW   128   /* R-SWA ring slots ([P3] const RING_WINDOW) */
#define KVQ_MAX_KV_HEADS  64
#define KVQ_MAX_CAPACITY  (1 << 24)   /* rows per (sequence, head): 32-bit offsets */
#define KVQ_ALL_SEQS      (-1)  /* `seq` value: one row for every sequence */

#define KVQ_OK         0
#define KVQ_EINVAL    (-1)  /* null pointer, bad shape or geometry, unsupported size */
#define KVQ_ECAPACITY (-2)  /* the rows would not fit in the cache's capacity */
#define KVQ_ESTATE    (-3)  /* wrong cache kind or state (e.g. ring prefill not recorded) */
#define KVQ_EDEVICE   (-4)  /* the HIP runtime refused a launch */

#define KVQ_KIND_F32  1
#define KVQ_KIND_Q8   2
#define KVQ_KIND_I8   3   /* per-row int8 ([P3] Int8Kv) */

/* Device buffers of a cache, for kvq_buffer_bytes(). */
#define KVQ_BUF_K     0   /* f32:  float [batch][n_live][capacity][128]            */
#define KVQ_BUF_V     1   /* f32:  float [batch][n_live][capacity][128]            */
#define KVQ_BUF_KQ    2   /* q8, i8: int8 [batch][n_live][capacity16 / 16][2][4][16][16],
                             tile-major (below); capacity16 = capacity rounded up
                             to a multiple of 16                             */
#define KVQ_BUF_KS    3   /* q8:   float [batch][n_live][capacity][4]  (one 16 B record per row);
                             i8:   float [batch][n_live][capacity]                 */
#define KVQ_BUF_VQ    4   /* q8, i8: int8 [batch][n_live][capacity][128]           */
#define KVQ_BUF_VS    5   /* q8, i8: float [batch][n_live][capacity]              */
#define KVQ_BUF_KCOL  6   /* q8:   float [batch][n_live][128]                      */
#define KVQ_BUF_VCOL  7   /* q8:   float [batch][n_live][128]                      */

/*
 * A per-layer KV cache of `batch` independent sequences ([P1] LayerKvCache,
 * one per sequence; [P3] BatchedRingCache for the batch dimension).
 *
 * Storage is head-major: every (sequence, live KV head) owns `capacity`
 * contiguous rows of 128 channels ([P1] module doc: one contiguous
 * [pos x head_dim] block per KV head).  Dead KV heads -- GQA groups whose Q
 * heads are all masked -- own no storage at all and get no work ([P1] module
 * doc: a masked head is neither stored nor computed); live heads are numbered
 * densely by live_slot.  The alive mask is fixed when the cache is created.
 *
 * f32 kind: K and V rows as float.
 * q8 kind ([P1] KvMode q8_2f): K rows as int8 codes with one f32 scale per
 * 32 channels, V rows as int8 codes with one f32 scale per row, and per
 * (sequence, live head) f32 column fields kcol/vcol that are 1 until the
 * freeze and the per-channel RMS afterwards.  A stored value is
 *   K^[p][d] = kq[p][d] * ks[p][d/32] * kcol[d],
 *   V^[p][d] = vq[p][d] * vs[p] * vcol[d].
 * i8 kind ([P3] Int8Kv, the per-row int8 route): K and V rows as int8 codes
 * with one f32 scale per row each (kq, ks, vq, vs; KVQ_BUF_KQ/VQ as for q8),
 *   K^[p][d] = kq[p][d] * ks[p],  V^[p][d] = vq[p][d] * vs[p].
 * K codes (both int8 kinds) are stored tile-major, in the order the matrix
 * cores read them: kq[p][d] of a (sequence, live head) is the byte at
 *   (p / 16) * 2048 + (d / 64) * 1024 + ((d / 16) % 4) * 256 + (p % 16) * 16
 *   + d % 16
 * of its capacity16 * 128-byte block; every other buffer is row-major.
 *
 * Fill it with kvq_cache_init(), then set the device pointers of the kind's
 * buffers (sizes from kvq_buffer_bytes(); every base must be 16-byte
 * aligned).  `len` and `frozen` point to caller-owned host arrays of `batch`
 * entries that the library keeps up to date.
 */
typedef struct kvq_cache {
    int32_t kind;            /* KVQ_KIND_F32, KVQ_KIND_Q8 or KVQ_KIND_I8 */
    int32_t batch;           /* sequences */
    int32_t n_kv_heads;      /* KV heads, dead ones included */
    int32_t head_dim;        /* 128 */
    int32_t capacity;        /* rows per (sequence, live head) */
    int32_t n_live;          /* live KV heads (set by kvq_cache_init) */
    int8_t  live_slot[KVQ_MAX_KV_HEADS];  /* storage slot of KV head g, -1 if dead */
    int32_t* len;            /* host [batch]: rows appended per sequence */
    uint8_t* frozen;         /* host [batch]: q8 column field frozen (0/1) */
    float*   k;              /* KVQ_BUF_K */
    float*   v;              /* KVQ_BUF_V */
    int8_t*  kq;             /* KVQ_BUF_KQ */
    float*   ks;             /* KVQ_BUF_KS */
    int8_t*  vq;             /* KVQ_BUF_VQ */
    float*   vs;             /* KVQ_BUF_VS */
    float*   kcol;           /* KVQ_BUF_KCOL */
    float*   vcol;           /* KVQ_BUF_VCOL */
} kvq_cache;

/*
 * R-SWA cursors of one sequence ([P3] RingCache fields prefill_len,
 * ring_len, ring_pos, decode_writes, lineage_epoch).  The sequence's rows are
 * the read-only reference block [0, prefill_len) followed by a ring of
 * KVQ_RING_WINDOW slots stored at rows [prefill_len, prefill_len + 128).
 */
typedef struct kvq_ring {
    int32_t prefill_len;     /* -1 until recorded */
    int32_t ring_len;        /* live ring slots, 0..128 */
    int32_t ring_pos;        /* next slot to overwrite once the ring is full */
    int32_t epoch;           /* lineage: advanced by a prefill and by a rollback that discards writes */
    int64_t writes;          /* ring writes since the prefill was recorded */
} kvq_ring;

/*
 * A checkpoint of one ring's cursors ([P3] RingCheckpoint): the cache,
 * sequence and stream it belongs to, and the cursors.  No K/V is copied.
 * `stream` is -1 for the ring of a sequence (rswa_checkpoint) and the
 * stream index for a stream of a shared reference (rswa_shared_checkpoint).
 */
typedef struct kvq_ring_checkpoint {
    const kvq_cache* cache;
    int32_t seq;
    int32_t prefill_len;
    int32_t ring_len;
    int32_t ring_pos;
    int32_t epoch;
    int32_t stream;
    int64_t writes;
} kvq_ring_checkpoint;

/*
 * Fill `c` for a new, empty cache: geometry, live-slot numbering from
 * `alive` (host [n_kv_heads], nonzero = live; NULL = all live), len[] = 0,
 * frozen[] = 0, device pointers NULL.  `len_host` and `frozen_host` are
 * caller-owned host arrays of `batch` entries and must outlive the cache.
 * Errors: KVQ_EINVAL (kind, head_dim != 128, batch < 1, capacity outside
 * 1..KVQ_MAX_CAPACITY, n_kv_heads outside 1..64, null arrays).
 */
int kvq_cache_init(kvq_cache* c, int kind, int batch, int n_kv_heads, int head_dim,
                   int capacity, const uint8_t* alive, int32_t* len_host,
                   uint8_t* frozen_host);

/* Bytes of device buffer `which` (KVQ_BUF_*) for this cache's geometry;
 * 0 for a buffer the kind does not use or an invalid argument. */
size_t kvq_buffer_bytes(const kvq_cache* c, int which);

/*
 * Bytes the stored rows occupy at the current lengths ([P1]
 * LayerKvCache::memory_bytes restricted to K/V storage): per (row, live
 * head) 2*4*128 = 1024 B for f32, 128 + 16 + 128 + 4 = 276 B for q8, plus
 * 2*4*128 B of column fields per live head of a frozen q8 sequence.
 */
size_t kvq_cache_bytes(const kvq_cache* c);

/*
 * kv_append_f32 -- [P1] LayerKvCache::append (f32 mode); [P3]
 * RingCache::record_prefill is this call followed by rswa_record_prefill.
 *
 * Appends `n_rows` rows to sequence `seq`: k_new/v_new are device float
 * [n_rows][n_kv_heads][128] (every KV head's values, dead ones included and
 * ignored).  Rows land at positions len[seq] .. len[seq]+n_rows-1 of every
 * live head; len[seq] += n_rows.
 * seq == KVQ_ALL_SEQS appends ONE row to every sequence: n_rows must be 1 and
 * k_new/v_new are [batch][n_kv_heads][128].
 * n_rows == 0 is a no-op.
 * Errors: KVQ_EINVAL (null, seq out of range, negative n_rows, missing
 * buffers), KVQ_ESTATE (not an f32 cache), KVQ_ECAPACITY (len + n_rows >
 * capacity for any affected sequence).
 */
int kv_append_f32(kvq_cache* c, int seq, int n_rows, const float* k_new,
                  const float* v_new, void* stream);

/*
 * kv_append_q8 -- [P1] LayerKvCache::append (q8_2f mode) with
 * [P1] quant_row, freezing through kv_freeze_col_and_requant exactly when
 * the page does.
 *
 * Same arguments and layout as kv_append_f32.  Each row is appended as if
 * alone, in order: at the start of appending a row to a sequence that holds
 * >= 64 rows and is not frozen, that sequence is frozen first (so rows
 * 0..63 are requantised and row 64 is the first one quantised against the
 * field).  A row r is quantised per live head as
 *   resid[d] = r[d] / col[d]            (col = 1 before the freeze),
 *   per group (32 channels for K, all 128 for V):
 *     s = max(max_d |resid[d]| / 127, 1e-12),
 *     code[d] = clamp(round_half_away(resid[d] / s), -127, 127),
 * in IEEE f32 with one rounding per operation.
 * Errors: as kv_append_f32, with KVQ_ESTATE for a non-q8 cache.
 */
int kv_append_q8(kvq_cache* c, int seq, int n_rows, const float* k_new,
                 const float* v_new, void* stream);

/*
 * kv_freeze_col_and_requant -- [P1] LayerKvCache::freeze_cols for one
 * sequence (seq == KVQ_ALL_SEQS: every sequence).
 *
 * For every live head, separately for K (group 32) and V (group 128), over
 * the n = len[seq] stored rows: x^ = f32(code) * scale; col[d] =
 * max(sqrtf((sum_p x^[p][d]^2) / n), 1e-6) with the sum taken in row order
 * in f32, multiply then add; every row is then requantised from x^ against
 * col.  Sets frozen[seq].  No-op for a sequence that is already frozen or
 * empty.  kv_append_q8 calls it by itself at row 64; calling it earlier
 * freezes the field over the rows stored so far.
 * Errors: KVQ_EINVAL (null, seq out of range), KVQ_ESTATE (not a q8 cache).
 */
int kv_freeze_col_and_requant(kvq_cache* c, int seq, void* stream);

/*
 * Bytes of workspace the decode calls need for this cache with n_q_heads
 * query heads (independent of the current lengths): partial softmax states
 * (max, sum, 128 accumulators per Q head of a group) for 8192 +
 * min(batch, 128) * n_live slots, rounded up to 256 bytes.  Its contents
 * need no initialisation.  Returns 0 on invalid arguments.
 */
size_t kvq_workspace_bytes(const kvq_cache* c, int n_q_heads);

/*
 * decode_attn_f32 -- single-query decode attention over every sequence of
 * an f32 cache: [P1] attend_group (GQA, each stored row read once per
 * group) and attend (per-head semantics); [P3] decode_attention_scalar_head
 * and fold (online softmax, never materialising the score row).
 *
 * q   device float [batch][n_q_heads][128]
 * out device float [batch][n_q_heads][128]
 * Q head h reads KV head g = h / (n_q_heads / n_kv_heads).  For a live g:
 *   out[b][h] = sum_p softmax_p(q[b][h] . K[b][g][p] / sqrt(128)) V[b][g][p]
 * over the len[b] stored rows, with no mask.  Q heads of dead groups, and
 * of sequences with no rows, get out = 0 ([P1] attend_group: stored == 0).
 * Results are f32; the summation order differs from the pages' serial loops.
 * ws/ws_bytes: device workspace of at least kvq_workspace_bytes().
 * Errors: KVQ_EINVAL (null, n_q_heads not a multiple of n_kv_heads, group
 * size n_q_heads/n_kv_heads not in {1, 2, 4, 8}, workspace too small),
 * KVQ_ESTATE (not an f32 cache).
 */
int decode_attn_f32(const kvq_cache* c, int n_q_heads, const float* q, float* out,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * decode_attn_q8 -- decode_attn_f32 over a q8 cache: [P1] attend (q8
 * branch) / attend_group, where a score is (1/sqrt(128)) * sum over K groups
 * of ks * <q (.) kcol, kq> and the output is (sum_p w_p vs_p vq_p) (.) vcol.
 * The query stays f32 (it is never quantised).  Same arguments, layout and
 * errors as decode_attn_f32 (KVQ_ESTATE for a non-q8 cache).
 */
int decode_attn_q8(const kvq_cache* c, int n_q_heads, const float* q, float* out,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * decode_attn_q8_noalloc -- decode_attn_q8 for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc): the same computation and kernels, with the
 * partial softmax states in a static device array of the library (64 MiB,
 * one per GPU, held until the process ends) instead of a caller's
 * workspace.  The call allocates nothing and frees nothing; the caller
 * still passes q and out (layouts as decode_attn_q8).  Every call on a GPU
 * shares that GPU's array, so calls that overlap on one GPU (different
 * streams, or host threads without ordering) race; calls ordered on one
 * stream do not.  Nothing in the array needs clearing between calls.
 * Errors: as decode_attn_q8, plus KVQ_EINVAL when the cache would need more
 * than 64 MiB of workspace (kvq_workspace_bytes() > 64 MiB: e.g. group
 * size 8 with min(batch, 128) x live heads > 7939), and KVQ_EDEVICE when
 * the array's device address cannot be looked up.
 */
int decode_attn_q8_noalloc(const kvq_cache* c, int n_q_heads, const float* q, float* out, void* stream);

/*
 * kv_append_i8 -- kv_append_f32 for an i8 cache: each row of each live head
 * is quantised as [P3] quantize_row_i8, separately for K and V:
 *   scale = max|x| / 127 (correctly rounded f32 division), or 1 for an
 *   all-zero row;  code = clamp(round_ties_even(x / scale), -127, 127)
 * with x / scale correctly rounded.  Same arguments and errors as
 * kv_append_f32 (KVQ_ESTATE for a cache of another kind).
 */
int kv_append_i8(kvq_cache* c, int seq, int n_rows, const float* k_new, const float* v_new, void* stream);

/*
 * decode_attn_i8 -- [P3] decode_attention_int8 over an i8 cache: each Q
 * head is quantised with quantize_row_i8 (codes and qscale, in f32); its
 * score against row p is (1/sqrt(128)) * qscale * ks[p] * <qcodes, kq[p]>
 * with the integer dot exact (|dot| <= 127 * 127 * 128); the softmax and the
 * value pass (weight * vs[p] * vq[p]) as decode_attn_f32.  Arguments,
 * layout, workspace and errors as decode_attn_f32 (KVQ_ESTATE for a cache
 * of another kind).
 */
int decode_attn_i8(const kvq_cache* c, int n_q_heads, const float* q, float* out,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * Options of decode_attn_f32_ex / decode_attn_q8_ex: the visible-row start,
 * logit soft-cap and learned sinks of [P2] LayerKvCache::attend_group_upto.
 *
 * first    host int32 [batch], or NULL for 0: sequence b attends rows
 *          [first[b], len[b]) only (a sliding window is first = len - W);
 *          first[b] >= len[b] is clamped to len[b] - 1, so at least one row
 *          stays visible.  Rows below first carry weight 0 exactly.
 * softcap  > 0: every scaled score s becomes softcap * tanh(s / softcap)
 *          (Gemma-2 soft-capping) before the softmax; 0 = off.
 * sinks    device float [n_q_heads], or NULL for none: one learned logit per
 *          Q head (same for every sequence).  The softmax treats it as one
 *          more logit that carries no value: it takes part in the maximum
 *          and contributes exp(sink - max) to the normaliser; it is not
 *          soft-capped.  A sequence with no rows still gives zeros.
 * The struct is read during the call only; `first` is copied into the
 * launch, so the caller may reuse it once the call returns.
 */
typedef struct kvq_decode_opts {
    const int32_t* first;
    float softcap;
    int32_t reserved;        /* 0 */
    const float* sinks;
} kvq_decode_opts;

/*
 * decode_attn_f32_ex / decode_attn_q8_ex -- decode_attn_f32 / decode_attn_q8
 * with the options above (opts NULL = no options: identical to the plain
 * calls).  Errors: as the plain calls, plus KVQ_EINVAL for a negative
 * first[b], a softcap that is negative or not finite, or reserved != 0.
 */
int decode_attn_f32_ex(const kvq_cache* c, int n_q_heads, const float* q, float* out,
                       const kvq_decode_opts* opts, void* ws, size_t ws_bytes, void* stream);
int decode_attn_q8_ex(const kvq_cache* c, int n_q_heads, const float* q, float* out,
                      const kvq_decode_opts* opts, void* ws, size_t ws_bytes, void* stream);

/*
 * rswa_record_prefill -- [P3] RingCache::record_prefill for sequence `seq`
 * of an f32 cache whose reference block has just been appended with
 * kv_append_f32, or of an i8 cache (the page's int8 mirror) appended with
 * kv_append_i8: prefill_len = len[seq], ring_len = ring_pos = writes = 0.
 * rings: host array [batch].  A prefill of 0 rows is allowed.
 * Errors: KVQ_EINVAL (null, seq out of range), KVQ_ESTATE (a q8 cache),
 * KVQ_ECAPACITY (len[seq] + 128 > capacity: no room for the ring).
 */
int rswa_record_prefill(kvq_cache* c, kvq_ring* rings, int seq);

/*
 * rswa_verify -- [P3] verify_attention: checks n_draft speculated tokens in
 * one call.  For every sequence b and draft i < n_draft, out[b][i]
 * is what the i-th of n_draft sequential rswa_decode steps fed with the draft
 * tokens 0..i would return: each Q head attends, with no mask, to the
 * reference rows, the ring as it would stand after draft tokens 0..i were
 * written (the oldest live slots evicted once it is full), and those draft
 * tokens.  Nothing is written: the cache and the ring cursors are unchanged
 * (accepting drafts is then rswa_decode, or a checkpoint / rollback).
 * On an i8 cache (the page's int8 mirror, its decode_attention being
 * decode_attention_int8) every draft row is quantised with quantize_row_i8
 * where the kernel reads it (nothing is stored), and every query per head.
 *
 * q        device float [batch][n_draft][n_q_heads][128]
 * k_draft, v_draft  device float [batch][n_draft][n_kv_heads][128]
 * out      device float [batch][n_draft][n_q_heads][128]
 * ws/ws_bytes  device workspace of at least kvq_verify_workspace_bytes().
 * n_draft x (n_q_heads / n_kv_heads) must be within 1..16.
 * Errors: KVQ_EINVAL (null, unaligned, bad counts, workspace too small),
 * KVQ_ESTATE (a q8 cache, a prefill not recorded, or a len that no longer
 * matches the cursors).
 */
int rswa_verify(const kvq_cache* c, const kvq_ring* rings, int n_q_heads, int n_draft, const float* q,
                const float* k_draft, const float* v_draft, float* out, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes rswa_verify needs with n_draft drafts, and rswa_shared_decode
 * with n_draft streams: partial states for n_draft x (n_q_heads / n_kv_heads)
 * queries per slot (at most 16), slots as kvq_workspace_bytes; 0 on invalid
 * arguments or more than 16 queries. */
size_t kvq_verify_workspace_bytes(const kvq_cache* c, int n_q_heads, int n_draft);

/*
 * rswa_checkpoint -- [P3] RingCache::checkpoint for sequence `seq`: copy its
 * cursors into *cp (host), taken before speculative decode steps.  O(1), no
 * device work.  Errors: KVQ_EINVAL (null, seq out of range), KVQ_ESTATE (a
 * q8 cache).
 */
int rswa_checkpoint(const kvq_cache* c, const kvq_ring* rings, int seq, kvq_ring_checkpoint* cp);

/*
 * rswa_rollback_to -- [P3] RingCache::rollback_to: discard every decode
 * step of sequence `seq` written since *cp was taken, by restoring ring_len,
 * ring_pos and writes (len[seq] = prefill_len + ring_len).  The dead slots
 * keep the discarded K/V and are never read.  A rollback that discards
 * writes advances the epoch, so checkpoints of the abandoned branch stop
 * matching.  Refused, with nothing changed, when the checkpoint belongs to
 * another cache or sequence, another prefill or epoch, is from the future,
 * or when the discarded writes overwrote a slot that was live at the
 * checkpoint (cp->ring_len + discarded > 128), or when *cp is a shared
 * stream's checkpoint (cp->stream != -1).  No device work.
 * Errors: KVQ_EINVAL (null, seq out of range), KVQ_ESTATE (a q8 cache, or
 * any refusal above).
 */
int rswa_rollback_to(kvq_cache* c, kvq_ring* rings, int seq, const kvq_ring_checkpoint* cp);

/*
 * kv_truncate_last -- [P1]/[P2] LayerKvCache::truncate_last for sequence
 * `seq` (or KVQ_ALL_SEQS): drop its last min(n_drop, len) rows, e.g. the
 * rejected tokens of a speculative step.  Host cursor only: the rows stay in
 * place and the next append overwrites them.  A q8 sequence keeps its frozen
 * column field, as the page keeps the fields.  Not for R-SWA sequences,
 * whose cursors rswa_rollback_to moves.
 * Errors: KVQ_EINVAL (null, seq out of range, n_drop < 0).
 */
int kv_truncate_last(kvq_cache* c, int seq, int n_drop);

/*
 * kv_trim_window -- [P2] LayerKvCache::trim_window_anchored for sequence
 * `seq`: drop the front rows a sliding-window layer of window w can never
 * read again.  *base (host, in/out) is the absolute position of the
 * sequence's row 0.  Nothing happens while len <= 2w, for w == 0, or on a q8
 * sequence before its freeze (the column field is computed over all stored
 * rows, so none may go before it).  Otherwise the rows from
 *   keep_from = min(base + len - (w + slack), anchor - (w + slack))  (>= 0)
 * on stay, the cut rounded down to a multiple of max(align, 1):
 *   d = (keep_from / align) * align - base   rows are dropped if d > 0,
 * the remaining rows move to the front of the sequence's storage in order
 * (kernels on `stream`), len -= d, *base += d.  anchor < 0 means none.
 * *dropped (may be NULL) receives d.  Windowed decodes of the trimmed
 * sequence (first = len - w) see the same rows as before.
 * seq == KVQ_ALL_SEQS trims every sequence by the same rule (same w, slack,
 * align and anchor): base is then a host array of batch entries, each the
 * position of that sequence's row 0 (in/out), and dropped (may be NULL) an
 * array of batch entries; all the moves run together, one launch per round
 * of at most d rows per sequence.
 * Errors: KVQ_EINVAL (null cache/base, seq out of range, any base, w, slack
 * or align < 0), KVQ_EDEVICE (launch failure).
 */
int kv_trim_window(kvq_cache* c, int seq, int64_t* base, int w, int slack, int align, int64_t anchor,
                   int* dropped, void* stream);

/*
 * rswa_decode -- one R-SWA decode step for every sequence of an f32 or i8
 * cache: [P3] attention() = write_decode_step() then decode_attention().
 * On an i8 cache (the page's int8 mirror) the step's K and V rows are
 * quantised into the ring slot with quantize_row_i8 and the attention is
 * decode_attention_int8 (query quantised per head, as decode_attn_i8).
 *
 * k_new, v_new  device float [batch][n_kv_heads][128]: this step's K/V
 * q             device float [batch][n_q_heads][128]
 * out           device float [batch][n_q_heads][128]
 * For each sequence b the step's K/V go to ring slot
 *   slot = ring_len            while ring_len < 128 (warm-up; ring_len += 1,
 *                              ring_pos = ring_len mod 128),
 *   slot = ring_pos            once full (ring_pos = (ring_pos + 1) mod 128),
 * i.e. to cache row prefill_len + slot, overwriting in place; then the query
 * attends, with NO causal mask, over rows [0, prefill_len + ring_len) --
 * the reference block and every live ring slot, itself included.  len[b]
 * becomes prefill_len + ring_len.  The reference rows are never written.
 * Errors: KVQ_EINVAL (null, bad group size, workspace too small),
 * KVQ_ESTATE (a q8 cache, or a sequence whose prefill was not recorded,
 * or whose len no longer matches its ring cursors),
 * KVQ_ECAPACITY (prefill_len + 128 > capacity).
 */
int rswa_decode(kvq_cache* c, kvq_ring* rings, int n_q_heads, const float* q,
                const float* k_new, const float* v_new, float* out,
                void* ws, size_t ws_bytes, void* stream);

/*
 * rswa_shared_record_prefill -- [P3] RingCache::record_prefill for a
 * reference block shared by n_streams decode streams (the prefix-shared
 * reference that [P3] batched_decode_attention leaves as a seam: streams
 * pointing at one reference block, each with its own ring).  Sequence `seq`
 * of an f32 or i8 cache holds the reference, just appended with
 * kv_append_f32 / kv_append_i8 (len[seq] rows); stream s's 128-slot ring is rows len[seq] + 128 s ..
 * len[seq] + 128 s + 127 of the same sequence.  Sets, for s < n_streams,
 * rings[s] = {prefill_len = len[seq], ring_len = ring_pos = writes = 0,
 * epoch + 1} and reserves the ring rows: len[seq] += 128 n_streams.
 * rings: host array [n_streams], the group's own (not indexed by sequence).
 * Errors: KVQ_EINVAL (null, seq out of range, n_streams outside 1..16),
 * KVQ_ESTATE (a q8 cache), KVQ_ECAPACITY (len[seq] + 128 n_streams >
 * capacity).
 */
int rswa_shared_record_prefill(kvq_cache* c, int seq, kvq_ring* rings, int n_streams);

/*
 * rswa_shared_decode -- one R-SWA decode step for each of the n_streams
 * streams that share sequence `seq`'s reference block.  Stream s's result is
 * what rswa_decode would give it alone: its step's K/V go to its ring slot
 * (the same cursor rules, row prefill + 128 s + slot), then its Q heads
 * attend, with no mask, over the reference rows and its own live ring slots
 * ([P3] batched_decode_attention: stream s attends reference ++ ring s).
 * The reference rows are read once for every stream's queries: n_streams x
 * (n_q_heads / n_kv_heads) <= 16 queries per KV head share each row read, a
 * dense contraction on the matrix cores.  On an i8 cache each step row is
 * quantised with quantize_row_i8 into its ring slot and the decode is the
 * int8 route.
 *
 * q, out        device float [n_streams][n_q_heads][128]
 * k_new, v_new  device float [n_streams][n_kv_heads][128]
 * ws/ws_bytes   at least kvq_verify_workspace_bytes(c, n_q_heads, n_streams).
 * Errors: KVQ_EINVAL (null, unaligned, seq out of range, n_streams x group
 * outside 1..16, workspace too small), KVQ_ESTATE (a q8 cache, group
 * not recorded, len[seq] no longer prefill + 128 n_streams, a stream with
 * another prefill or corrupt cursors).  Nothing is written on error.
 */
int rswa_shared_decode(kvq_cache* c, int seq, kvq_ring* rings, int n_streams, int n_q_heads, const float* q,
                       const float* k_new, const float* v_new, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * rswa_shared_checkpoint -- [P3] BatchedRingCache::checkpoint: the cursors
 * of stream `s` (0 <= s < n_streams) of the shared group recorded on
 * sequence `seq` (rswa_shared_record_prefill), copied into *cp (host), with
 * cp->stream = s.  Each stream is checkpointed on its own.  O(1), no device
 * work.
 * Errors: KVQ_EINVAL (null, seq or s out of range, n_streams outside
 * 1..16), KVQ_ESTATE (a q8 cache, a group not recorded, or len[seq] not
 * prefill + 128 n_streams).
 */
int rswa_shared_checkpoint(const kvq_cache* c, int seq, const kvq_ring* rings, int n_streams, int s,
                           kvq_ring_checkpoint* cp);

/*
 * rswa_shared_rollback_to -- [P3] BatchedRingCache::rollback_to: stream s
 * of the shared group on sequence `seq` goes back to *cp under the
 * lossless contract of rswa_rollback_to (ring_len, ring_pos and writes
 * restored; a rollback that discards writes advances the stream's epoch).
 * No other stream and no row of the cache changes (len[seq] stays prefill
 * + 128 n_streams: the rings' rows stay reserved), and nothing runs on the
 * device.  Refused, with nothing changed, when the checkpoint belongs to
 * another cache, sequence or stream, another prefill or epoch, is from the
 * future, or would need a ring row the discarded writes overwrote
 * (cp->ring_len + discarded > 128).
 * Errors: KVQ_EINVAL (null, seq or s out of range, n_streams outside
 * 1..16), KVQ_ESTATE (a q8 cache, a group not recorded, len[seq] not
 * prefill + 128 n_streams, or any refusal above).
 */
int rswa_shared_rollback_to(kvq_cache* c, int seq, kvq_ring* rings, int n_streams, int s,
                            const kvq_ring_checkpoint* cp);

/* Message of the last failed call on this thread ("" if none). */
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
