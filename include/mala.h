/*
 * mala.h -- C ABI of libmala.so: MassAlloc Attention (MALA) on AMD Instinct
 * MI355X (gfx950).
 *
 * MALA is causal softmax attention that still scores every legal causal tile
 * (QK) but gates the post-score work of each tile on the tile's normalized
 * contribution.  Source: "MassAlloc Attention: Let Attention Allocate Its Own
 * Compute", digest page at agihunt.info (arXiv 2609.32712).  Its paragraphs
 * are cited by topic:
 *   threshold paragraph  -- the per-tile test of the largest per-key
 *                           contribution ratio against tau/Lq, Lq = number of
 *                           causally visible keys of the query row;
 *   forward paragraph    -- test against the running online-softmax
 *                           normalizer, block vote, diagonal-to-early visit
 *                           order, first legal tile always kept, lse written;
 *   backward paragraph   -- test against the final log-normalizer, nested
 *                           support, no stored mask;
 *   savings paragraph    -- what a skipped tile saves; tau -> 0 gives full
 *                           attention; no attention matrix or mask stored.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensors are DEVICE pointers to densely packed row-major arrays; the
 *    library allocates nothing, keeps no pointer after returning and never
 *    synchronizes the device.  The caller owns every buffer (including the
 *    workspace) and must keep it alive until the work queued on `stream` has
 *    finished.
 *  - `stream` is a hipStream_t (NULL: the default stream).  All work is queued
 *    on it in order; calls are asynchronous.
 *  - Element type `dtype`: MALA_BF16 tensors hold bfloat16 values, MALA_F32
 *    tensors hold float.  lse and statistics are always float / int32.
 *    Arithmetic is fp32 (bf16 MFMA products accumulated in fp32).
 *  - Scores are s_ij = scale * <q_i, k_j>; scale <= 0 selects 1/sqrt(d).
 *    lse is the natural-log normalizer: lse_i = ln sum_{kept j} exp(s_ij).
 *  - tau >= 0 (finite or +inf).  tau = 0 selects the ungated instantiation
 *    (full causal attention, every legal tile kept).  tau = +inf keeps only
 *    the tiles forward must keep (those visited while a row is still empty)
 *    and nothing in backward.
 *  - Errors: every argument is validated before anything is queued; on error
 *    nothing is queued, the status is returned and mala_last_error() (per
 *    thread) describes it.  A HIP launch failure returns MALA_ERR_HIP.
 *  - Thread safety: calls may be made concurrently from several host threads.
 *
 * Supported shapes (anything else returns MALA_ERR_UNSUPPORTED)
 *  - prefill (fwd/bwd): H % Hkv == 0 (else MALA_ERR_INVALID_ARG); L >= 1
 *      (ragged L allowed), L*d < 2^31 (Lcap*d for chunked prefill) and
 *      B*H*L*d < 2^40;
 *      MALA_BF16 with d = 128 and tile {128, 64} (grouped K/V heads allowed);
 *      MALA_F32  with d = 64  and tile {64, 64} (H == Hkv only).
 *  - decode: Hq % Hkv == 0 (else MALA_ERR_INVALID_ARG) with G = Hq/Hkv one of
 *      1, 2, 4, 8; MALA_BF16, d = 128, bk = 64, split_keys a positive multiple
 *      of bk.
 */
#ifndef MALA_H
#define MALA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MALA_OK = 0,
    MALA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, tau < 0 or NaN, short workspace */
    MALA_ERR_UNSUPPORTED = -2, /* valid request outside the supported shapes listed above           */
    MALA_ERR_HIP = -3          /* a HIP runtime call or kernel launch failed                         */
} mala_status;

typedef enum { MALA_BF16 = 0, MALA_F32 = 1 } mala_dtype;

/* Tile shape: bq query rows (one vote block) by bk keys. */
typedef struct {
    int bq;
    int bk;
} mala_tile;

/*
 * Optional per-call statistics; every pointer may be NULL (not written).
 * Prefill (fwd or bwd), nqb = ceil(L/bq), ntiles = ceil(L/bk),
 * words = ceil(ntiles/32):
 *   kept      int32 [B, H, nqb]         tiles kept per query block
 *   legal     int32 [B, H, nqb]         legal (tested) tiles per query block
 *   keep_bits uint32 [B, H, nqb, words] bit (t % 32) of word t/32 = tile t kept
 * Decode, nsplit = ceil(Lk/split_keys), tps = split_keys/bk, words = ceil(tps/32),
 * V = Hkv * G/rows_per_vote vote groups per sequence ([B, Hkv, nsplit] when a
 * whole KV group votes together):
 *   kept, legal int32 [B, V, nsplit];  keep_bits uint32 [B, V, nsplit, words],
 *   bit t = tile t of the partition (tile 0 starts at the partition start).
 *   keep_bits_dkdv uint32 [B, H, nqb, words], mala_bwd only: the tiles the
 *             dK/dV pass actually processed (the dQ pass writes keep_bits and
 *             hands the same decisions to the dK/dV pass); the two must agree
 *             bit for bit.  The call clears it (with a kernel) and the dK/dV
 *             pass sets its bits.
 *   test_stat float, bf16 only (MALA_ERR_UNSUPPORTED on the fp32 path): log2
 *             of each tested tile's statistic T, i.e. the largest margin
 *             c*max_j s_ij - (running log2 max + log2 l + log2 tau - log2 Lq_i)
 *             of a voting row, c = scale*log2(e), s_ij = <q_i, k_j>; the tile
 *             is kept iff it is >= 0 (up to fp32 rounding of the two forms).
 *             +inf for an empty running state, -inf when no row votes (tau =
 *             +inf), NaN at tau = 0 (no test).  Forward (and mala_fwd_chunk):
 *             the running state before the tile, [B, H, nqb, ceil(Lk/bk)];
 *             mala_bwd (dQ pass): the final lse, [B, H, nqb, ntiles]; decode:
 *             per vote group, [B, V, nsplit, split_keys/bk].  Entries of
 *             tiles that are not tested are not written.
 * Every call only launches kernels on `stream` (no allocation, no memset, no
 * synchronization), so it can be captured in a HIP graph; events in
 * mala_stats are recorded with hipEventRecord and are for eager calls.
 *   events    up to 4 hipEvent_t handles (NULL entries skipped), recorded on
 *             `stream` around the call's kernels: mala_fwd and mala_decode
 *             record events[0] before and events[1] after their kernels;
 *             mala_bwd records events[0] before the row-state kernel,
 *             events[1] before the dQ pass, events[2] before the dK/dV pass
 *             and events[3] after it.  For per-kernel timing by the caller.
 * These are debug/measurement outputs: the library never reads them back and
 * backward does not consume anything forward wrote here.
 */
typedef struct {
    int32_t* kept;
    int32_t* legal;
    uint32_t* keep_bits;
    uint32_t* keep_bits_dkdv;
    void* events[4];
    float* test_stat;
} mala_stats;

/*
 * mala_fwd -- gated forward (forward paragraph, threshold paragraph).
 *
 * q: [B, H, L, d]; k, v: [B, Hkv, L, d], query head h reading K/V head
 * h / (H/Hkv) (grouped-query attention; Hkv == H is ordinary multi-head).
 * o: [B, H, L, d] (same dtype).  lse: float [B, H, L].
 * For each query block of bq rows, key tiles t = jmax .. 0 (diagonal first)
 * are scored; row i of the block votes to keep tile t iff its running state
 * is empty or max_j exp(s_ij - m_i)/l_i >= tau/(i+1) over its visible keys
 * (m_i, l_i: running max and normalizer before the tile); the tile is kept
 * for the whole block iff any row votes keep; only kept tiles load V and
 * update (m, l, acc).  o = acc/l, lse = m + ln l.
 */
mala_status mala_fwd(const void* q, const void* k, const void* v,
                     int B, int H, int Hkv, int L, int d, mala_dtype dtype,
                     float tau, mala_tile tile, float scale,
                     void* o, float* lse, mala_stats* stats, void* stream);

/*
 * mala_fwd_chunk -- gated forward of a query chunk against a key/value cache
 * (chunked prefill; threshold paragraph: one test for training, prefill and
 * decoding, with Lq the row's count of visible keys).
 *
 * q: [B, H, Lq, d], row i at key position P + i.  kcache, vcache:
 * [B, Hkv, Lcap, d]; rows 0 .. P + Lq - 1 are valid (the cache holds the P
 * earlier keys and the chunk's own keys at P .. P + Lq - 1); Lcap >= P + Lq.
 * Query head h reads K/V head h / (H/Hkv).  Row i sees keys 0 .. P + i and
 * Lq_i = P + i + 1.  Query blocks of bq rows are counted from the chunk
 * start, key tiles of bk keys from key 0; each block visits its tiles from the
 * one holding its last row's key back to key 0 with the forward's test and
 * update.  With P = 0 and Lcap = Lq this is mala_fwd.  o: [B, H, Lq, d],
 * lse: float [B, H, Lq].  Statistics as for mala_fwd with
 * ntiles = ceil((P + Lq)/bk).  bf16, d = 128, tile {128, 64} only.
 * Errors: P < 0 or P + Lq > Lcap -> MALA_ERR_INVALID_ARG; other dtypes ->
 * MALA_ERR_UNSUPPORTED.
 */
mala_status mala_fwd_chunk(const void* q, const void* kcache, const void* vcache,
                           int B, int H, int Hkv, int Lq, int P, int Lcap, int d, mala_dtype dtype,
                           float tau, mala_tile tile, float scale,
                           void* o, float* lse, mala_stats* stats, void* stream);

/* Workspace bytes mala_bwd needs for these sizes (0 for invalid sizes). */
size_t mala_bwd_workspace_size(int B, int H, int L, int d, mala_dtype dtype, mala_tile tile);

/*
 * mala_bwd -- gated backward (backward paragraph).
 *
 * Inputs q, o, dout: [B, H, L, d]; k, v: [B, Hkv, L, d] (as in mala_fwd);
 * lse: float [B, H, L] -- o and lse exactly as mala_fwd wrote them (the
 * ordinary attention state; no mask).  Outputs dq: [B, H, L, d], dk, dv:
 * [B, Hkv, L, d], fully overwritten; with grouped heads dk and dv sum the
 * contributions of the H/Hkv query heads that share a K/V head.
 * With P_ij = exp(s_ij - lse_i), a tile (query block, key tile) is kept iff
 * some row has a visible key with P_ij >= tau/(i+1) (no forced keep).  Kept
 * tiles contribute dV += P^T dO, dS = P o (dO V^T - D) with
 * D_i = sum_c dO_ic O_ic, dQ += scale dS K, dK += scale dS^T Q; skipped tiles
 * contribute nothing.  tile must equal the forward's.
 * workspace: device buffer of at least mala_bwd_workspace_size(...) bytes,
 * 256-byte aligned, contents ignored on entry.  It holds three per-row fp32
 * arrays [B, H, L] (D, base-2 lse, threshold) and the decision bits
 * [B, H, nqb, ceil(ntiles/32)] that the dQ pass hands to the dK/dV pass within
 * this call (nothing is kept between calls).
 */
mala_status mala_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, int B, int H, int Hkv, int L, int d, mala_dtype dtype,
                     float tau, mala_tile tile, float scale,
                     void* dq, void* dk, void* dv, mala_stats* stats,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes mala_decode and mala_decode_seeded need for these sizes (0
 * for invalid sizes): the partition states, B*Hq*nsplit*(d+2) floats with
 * nsplit = ceil(Lk/split_keys), rounded up to 256 bytes; when nsplit > 1 and
 * split_keys/64 <= 256, plus the states of the newest partition's 64-key
 * tiles, B*Hq*(split_keys/64)*(d+2) floats rounded up to 256 bytes (used by
 * mala_decode_seeded only; mala_decode needs the first part).
 */
size_t mala_decode_workspace_size(int B, int Hq, int Hkv, int Lk, int d, int split_keys);

/*
 * mala_decode -- one new query token per sequence against a KV cache, with
 * the same test (threshold paragraph: one tau for training and decoding).
 *
 * q: [B, Hq, d] (query at position Lk-1).  kcache, vcache: [B, Hkv, Lcap, d];
 * rows 0 .. Lk-1 are valid (row Lk-1 holds the new token).  o: [B, Hq, d];
 * lse: float [B, Hq] or NULL.  Query head h uses KV head h / (Hq/Hkv).
 * Split-KV: keys are cut into partitions [p*split_keys, min((p+1)*split_keys, Lk));
 * each partition is cut into bk-key tiles from its start and visited last tile
 * first with its own running state (so its first visited tile is kept); Lq =
 * Lk.  Partition states are merged exactly.
 * Votes: the G = Hq/Hkv query heads of a KV group share every K/V tile load
 * and vote in groups of rows_per_vote consecutive heads (0 means G: the whole
 * group votes together, so a skipped tile saves its V read; 1: every query
 * head votes alone).  A tile is kept for a vote group iff one of its heads
 * votes keep; only the heads of a group that keeps it update their state, and
 * V is read iff some group keeps it.  rows_per_vote must divide G
 * (MALA_ERR_INVALID_ARG otherwise).
 * Statistics are per vote group: kept, legal [B, Hkv * G/rows_per_vote,
 * nsplit] and keep_bits [B, Hkv * G/rows_per_vote, nsplit, ceil(split_keys /
 * bk / 32)], group j of KV head g at index g * (G/rows_per_vote) + j.
 * workspace: at least mala_decode_workspace_size(...) bytes, 256-byte aligned.
 */
mala_status mala_decode(const void* q, const void* kcache, const void* vcache,
                        int B, int Hq, int Hkv, int Lk, int Lcap, int d, mala_dtype dtype,
                        float tau, int split_keys, int bk, int rows_per_vote, float scale,
                        void* o, float* lse, mala_stats* stats,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * mala_decode_seeded -- mala_decode with seeded partitions (threshold and
 * forward paragraphs: a tile is tested against a normalizer established on
 * the more recent keys; seeding carries that normalizer across split-KV
 * partitions).  Arguments, shapes, workspace and errors are mala_decode's.
 *
 * Tiles are the bk-key tiles counted from key 0; jd = (Lk-1)/bk is the tile
 * of the newest key.  Partition p (p = 0 newest) holds tiles
 * max(0, jd - (p+1)*tps + 1) .. jd - p*tps, tps = split_keys/bk, and is
 * visited newest tile first.  Partition 0 starts from an empty state (its
 * first visited tile is kept), exactly as a mala_decode partition.  Every
 * older partition is tested against partition 0's final normalizer plus its
 * own kept keys, and keeps nothing by force; its output state holds only its
 * own kept keys, and the partitions' states are merged exactly.  Partition
 * 0 runs first: with older partitions (and tps <= 256) as the states of its
 * tiles, formed in parallel, followed by a replay of its walk over them (the
 * same test and merge, so the same decisions up to floating-point rounding
 * of the merge order); otherwise tile by tile.  The older partitions follow
 * (tau = 0: one launch, every tile kept).  Statistics as for mala_decode with nsplit = ceil(Lk /
 * split_keys) partitions in this order; bit t of partition p = its t-th tile
 * from the oldest.  events[0] is recorded before the first launch and
 * events[1] after the merge.
 */
mala_status mala_decode_seeded(const void* q, const void* kcache, const void* vcache,
                               int B, int Hq, int Hkv, int Lk, int Lcap, int d, mala_dtype dtype,
                               float tau, int split_keys, int bk, int rows_per_vote, float scale,
                               void* o, float* lse, mala_stats* stats,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * mala_decode_noalloc -- mala_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It takes mala_decode's arguments without the workspace
 * and computes exactly what mala_decode computes (the same kernels, bit for
 * bit), keeping the split partial states in a static device array of
 * MALA_DECODE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends.  It calls no hipMalloc or hipFree; its
 * first call on a device (with that device current) looks the array's address
 * up with hipGetSymbolAddress and keeps it.
 *
 * Limit: the partials need B * Hq * ceil(Lk/split_keys) * (d + 2) * 4 bytes
 * (8.8 MB for 16 sequences x 32 heads x 131,073 keys with 4096-key splits);
 * a call needing more than MALA_DECODE_NOALLOC_SCRATCH_BYTES returns
 * MALA_ERR_UNSUPPORTED before anything is queued.  Nothing in the array needs
 * clearing: every call writes each partial it reads.
 * Concurrency: every call on one GPU shares that GPU's array, so calls that
 * overlap on one GPU (on different streams, or from several host threads
 * without ordering) race; serialize them, e.g. on one stream.  The call runs
 * on the current device, to which `stream` must belong.
 */
#define MALA_DECODE_NOALLOC_SCRATCH_BYTES (16u << 20)
mala_status mala_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                                int B, int Hq, int Hkv, int Lk, int Lcap, int d, mala_dtype dtype,
                                float tau, int split_keys, int bk, int rows_per_vote, float scale,
                                void* o, float* lse, mala_stats* stats, void* stream);

/* Static description of a status code. */
const char* mala_status_string(mala_status status);
/* Message of the last failing call on this host thread ("" if none). */
const char* mala_last_error(void);
/* ABI version (major * 100 + minor). */
int mala_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MALA_H */
