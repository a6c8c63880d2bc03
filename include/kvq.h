/*
 * kvq.h -- C ABI of the quantized KV-cache library for MI355X (gfx950).
 *
 * The library writes new K/V vectors into a quantized cache (quantize, then
 * scatter to slots) and runs decode / chunked-prefill attention that
 * dequantizes the cache on the fly.  Every entry point is asynchronous: it
 * validates its arguments on the host, enqueues its kernels on the caller's
 * HIP stream and returns.  Nothing is enqueued when an argument is rejected.
 * The library never allocates, frees or synchronizes; every buffer is owned by
 * the caller and lives in device memory unless a comment says otherwise.
 * Scalars that change from step to step (start position, kv_len) are device
 * int32 values read by the kernels, so a captured step replays correctly.
 *
 * Page references (titles and sections of the pages this follows):
 *   [PR24473]  pytorch/executorch pull request 24473, Summary
 *   [PR20351]  pytorch/executorch pull request 20351 (gemma4_31b on the CUDA
 *              backend), commit notes on index_copy_, the per-tile causal
 *              upper bound and the kv_len bound
 *   [IQC]      IndexerQuantCache (ops-transformer): function description,
 *              parameter table, constraints
 *   [ABADDON]  abaddon 0.2.0-rc.1, src/attention_cache/mod.rs, trait KvCache
 *
 * Layouts (row-major, innermost last):
 *   new K/V x        [B, H, T, D]   bf16 or fp32; D contiguous, other strides
 *                                   given in elements     ([ABADDON] append)
 *   cache codes      [B, H, S, row_bytes] uint8           ([PR20351] positions
 *                                   on dim 2, nibble packing on the last dim)
 *   cache scales     INT8_TH/UINT4_TH: float [B, H, S]
 *                    FP8E4M3_B32, FP8E5M2_B32, INT8_B32: float [B, H, S, D/32]
 *                    MXFP4_B32, MXFP8_B32, MXFP4E1M2_B32: uint8 E8M0 [B, H, S, D/32]
 *   cache zps        INT8_TH/UINT4_TH: int8 [B, H, S]; NULL for block modes
 *   q / out          [B, Hq, Lq, D] contiguous             ([ABADDON]
 *                                   forward_attention)
 *   row_bytes        D/2 for UINT4_TH, MXFP4_B32 and MXFP4E1M2_B32 (two codes per byte,
 *                    element 2i in the low nibble), D for the other modes.
 *
 * Device error flags: entry points that take `int32_t* err_flags` (device,
 * nullable) OR these bits into it when the data (not the arguments) is out of
 * range; the offending token is skipped or the bound clamped, never written
 * out of bounds.  The caller clears the word and reads it when it wants to.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
    KVQ_OK = 0,
    KVQ_ERR_NULL = 1,        /* a required pointer is NULL */
    KVQ_ERR_SHAPE = 2,       /* a size or stride is out of the supported range */
    KVQ_ERR_DTYPE = 3,       /* dtype / quantization mode not valid for the call */
    KVQ_ERR_UNSUPPORTED = 4, /* valid request this build does not run (never degraded) */
    KVQ_ERR_WORKSPACE = 5,   /* workspace missing or too small */
    KVQ_ERR_LAUNCH = 6       /* the HIP runtime refused a launch */
} kvq_status;

typedef enum kvq_qmode {
    KVQ_INT8_TH = 0,      /* per token-head affine int8, fp32 scale, int8 zp [PR24473] */
    KVQ_UINT4_TH = 1,     /* per token-head affine 4-bit, two codes per byte [PR20351] */
    KVQ_FP8E4M3_B32 = 2,  /* per-32 block FP8-E4M3FN + fp32 scale, amax/448 [IQC] */
    KVQ_MXFP4_B32 = 3,    /* per-32 block FP4-E2M1 + E8M0 scale [IQC] */
    KVQ_MXFP8_B32 = 4,    /* per-32 block FP8-E4M3FN + E8M0 scale (MX-FP8 mode) [IQC] */
    KVQ_FP8E5M2_B32 = 5,  /* per-32 block FP8-E5M2 + fp32 scale, amax/57344 [IQC] */
    KVQ_INT8_B32 = 6,     /* per-32 block symmetric int8 in a uint8 plane + fp32 scale, amax/127 [IQC] */
    KVQ_MXFP4E1M2_B32 = 7 /* per-32 block FP4-E1M2 + E8M0 scale (MX-FP4 mode, FLOAT4_E1M2 cache) [IQC]:
                             sign, one exponent bit of bias 0, two mantissa bits, so magnitude code
                             k (0..7) is worth k / 2; Q_MAX 3.5, emax 1; packed as MXFP4_B32 */
} kvq_qmode;

typedef enum kvq_dtype { KVQ_F32 = 0, KVQ_BF16 = 1 } kvq_dtype;

#define KVQ_FLAG_SLOT_RANGE 1    /* a slot outside [-1, n_slots): token skipped */
#define KVQ_FLAG_KVLEN 2         /* kv_len outside [Lq, n_slots]: clamped */
#define KVQ_FLAG_POS_CAPACITY 4  /* full-context position >= capacity: not written */

#define KVQ_NO_CAUSAL_SKIP 1u    /* prefill: scan all KV tiles below kv_len
                                    (the per-tile causal bound switched off) */

#define KVQ_MX_SCALE_OCP 1u      /* quantize, MX modes: E8M0 scale 2^(floor(log2 amax)
                                    - emax) (emax 2 for E2M1, 1 for E1M2, 8 for E4M3; elements
                                    past Q_MAX saturate) instead of the smallest
                                    power of two >= amax / Q_MAX.  The reading of
                                    [IQC]'s round_scale = false. */

/* One quantized cache (K or V).  Caller-owned device planes, see layouts. */
typedef struct kvq_cache {
    int32_t qmode;      /* kvq_qmode */
    int32_t batch;      /* B */
    int32_t heads;      /* KV heads H */
    int32_t n_slots;    /* S, slots per (b, h) */
    int32_t head_dim;   /* D */
    void* codes;
    void* scales;
    int8_t* zps;        /* NULL for the block modes */
} kvq_cache;

/* Human-readable name of a status code (static storage). */
const char* kvq_status_string(kvq_status s);

/* Bytes of each plane of a cache with these sizes ([ABADDON] memory_bytes).
 * Any output pointer may be NULL.  KVQ_ERR_SHAPE for non-positive sizes, odd
 * D in the 4-bit modes or D % 32 != 0 in the block modes. */
kvq_status kvq_cache_bytes(int qmode, int B, int H, int n_slots, int D,
                           size_t* codes_bytes, size_t* scales_bytes, size_t* zps_bytes);

/* Quantize new vectors and scatter them into cache slots.
 *   [PR24473] int8 per token and head, affine asymmetric, fp32 scale + int8
 *   zero point, written through the slot indices;  [PR20351] static scatter
 *   along the position dim, nibble-packed 4-bit codes;  [IQC] per-32 block
 *   formula scale = max|x_g| / Q_MAX, q = round(x / scale), slot -1 skipped.
 * x: [B, H, T, D] in x_dtype with element strides (stride_b, stride_h,
 *   stride_t), D contiguous; B, H, D must equal the cache's.
 * slot_mapping: int32, token (b, t) uses slot_mapping[b*slot_stride_b + t];
 *   slot_stride_b = 0 shares one row of T slots across the batch.  -1 skips
 *   the token; any other value outside [0, n_slots) skips it and sets
 *   KVQ_FLAG_SLOT_RANGE.  Valid slots of one call must be distinct (a
 *   repeated slot leaves either token's row, unspecified which).
 * Every head of the token is written: codes, scale and (affine modes) zero
 *   point of row (b, h, slot).  All other bytes of the cache are untouched.
 * Rounding: round half to even, IEEE fp32 division, no contraction; codes,
 *   scales and zero points are bit-exact with the documented formulas.
 * Limits: T >= 0 (T == 0 enqueues nothing), D % 8 == 0 and D <= 8192
 *   (affine modes), D % 32 == 0 and D <= 8192 (block modes); B*H*T*D < 2^34
 *   elements per call (else KVQ_ERR_SHAPE; split the call along T). */
kvq_status kvq_quant_scatter(const void* x, int x_dtype, int B, int H, int T, int D,
                             int64_t stride_b, int64_t stride_h, int64_t stride_t,
                             const int32_t* slot_mapping, int64_t slot_stride_b,
                             const kvq_cache* cache, int32_t* err_flags, void* stream);

/* kvq_quant_scatter with quantization options: flags = 0 is kvq_quant_scatter;
 * KVQ_MX_SCALE_OCP selects the floor rule for the E8M0 scale of MXFP4_B32, MXFP4E1M2_B32 and
 * MXFP8_B32 caches.  KVQ_ERR_UNSUPPORTED for unknown bits or for an option the
 * cache's mode does not have. */
kvq_status kvq_quant_scatter_flags(const void* x, int x_dtype, int B, int H, int T, int D,
                                   int64_t stride_b, int64_t stride_h, int64_t stride_t,
                                   const int32_t* slot_mapping, int64_t slot_stride_b,
                                   const kvq_cache* cache, unsigned flags, int32_t* err_flags,
                                   void* stream);

/* The K and V update of one step in a single launch ([PR24473] writes new
 * keys and values into their two caches through the same slot indices):
 * exactly kvq_quant_scatter(xk, ..., k_cache) followed by
 * kvq_quant_scatter(xv, ..., v_cache).  xk and xv share dtype, sizes and
 * strides; the two caches must have the same mode and sizes (else
 * KVQ_ERR_SHAPE).  Bad slots set KVQ_FLAG_SLOT_RANGE as above. */
kvq_status kvq_quant_scatter_kv(const void* xk, const void* xv, int x_dtype, int B, int H, int T, int D,
                                int64_t stride_b, int64_t stride_h, int64_t stride_t,
                                const int32_t* slot_mapping, int64_t slot_stride_b,
                                const kvq_cache* k_cache, const kvq_cache* v_cache,
                                int32_t* err_flags, void* stream);

/* The K and V update of a full-context cache in one launch, its slots
 * derived on the device: exactly kvq_positions_full(start_pos, T, n_slots,
 * slots, NULL, err_flags) followed by kvq_quant_scatter_kv(xk, xv, ...,
 * slots, 0, k_cache, v_cache, err_flags) ([PR20351] commit notes: the new
 * token's K and V go to the cache at the device-side input position, so a
 * captured step needs no host value).  Token t of every batch row goes to
 * slot p = *start_pos + t; a negative *start_pos writes nothing and sets
 * KVQ_FLAG_SLOT_RANGE, a p >= n_slots writes nothing for that token and sets
 * KVQ_FLAG_POS_CAPACITY.  start_pos: device int32 scalar.  Arguments, limits
 * and errors otherwise as kvq_quant_scatter_kv (KVQ_ERR_NULL for a null
 * start_pos when T > 0). */
kvq_status kvq_quant_scatter_kv_full(const void* xk, const void* xv, int x_dtype, int B, int H, int T, int D,
                                     int64_t stride_b, int64_t stride_h, int64_t stride_t,
                                     const int32_t* start_pos, const kvq_cache* k_cache,
                                     const kvq_cache* v_cache, int32_t* err_flags, void* stream);

/* Write slots for positions p = *start_pos + t, t in [0, T), attention-sink
 * layout ([PR24473]): n_slots = sink_size + window, slot = p for p < sink_size,
 * else sink_size + (p - sink_size) mod window.  slot_mapping_out: int32 [T].
 * cache_positions: int32 [sink_size + window], in/out, -1 = empty; receives
 * cache_positions[slot] = p (the latest position wins when a chunk wraps).
 * A call with more tokens than the window writes them as if one after
 * another: a token whose slot a later token of the same call takes again
 * gets slot -1 (not written), so the scatter never sees a slot twice.
 * start_pos is a device int32 scalar; a negative value writes slot -1 for
 * every token and sets KVQ_FLAG_SLOT_RANGE.  sink_size >= 0, window >= 1. */
kvq_status kvq_positions_with_sink(const int32_t* start_pos, int T, int sink_size, int window,
                                   int32_t* slot_mapping_out, int32_t* cache_positions,
                                   int32_t* err_flags, void* stream);

/* Ring / sliding-window layout ([PR24473]): the sink layout with sink_size 0,
 * slot = p mod window. */
kvq_status kvq_positions_ring(const int32_t* start_pos, int T, int window,
                              int32_t* slot_mapping_out, int32_t* cache_positions,
                              int32_t* err_flags, void* stream);

/* Full-context layout ([PR24473]): slot = p; a position >= capacity is
 * rejected (slot -1, KVQ_FLAG_POS_CAPACITY) instead of written.
 * cache_positions may be NULL. */
kvq_status kvq_positions_full(const int32_t* start_pos, int T, int capacity,
                              int32_t* slot_mapping_out, int32_t* cache_positions,
                              int32_t* err_flags, void* stream);

/* Additive mask for a ring/sink cache ([PR24473]: those caches build an
 * additive float mask): mask_out[r, s] (fp32 [Lq, n_slots]) is 0 when the
 * slot's position cp = cache_positions[s] is visible to query position
 * qp = *start_pos + r, i.e. cp >= 0, cp <= qp and (cp < sink_size or
 * qp - cp < window), and -inf otherwise.  KVQ_ERR_SHAPE unless
 * sink_size + window == n_slots (the cache is its sink plus its window; a
 * full-context cache is sink_size 0, window n_slots). */
kvq_status kvq_build_mask(const int32_t* cache_positions, int n_slots, const int32_t* start_pos,
                          int Lq, int sink_size, int window, float* mask_out, void* stream);

/* Workspace bytes kvq_sdpa_decode needs for these sizes: a counter region
 * (one 4-byte ticket per (batch, kv head), rounded up to 256 bytes), then the
 * partial softmax states of the split-K pass.  It is an upper bound valid on
 * any device and for every cache mode (the split count of a launch depends on
 * how many workgroups the device keeps resident); needs no device.  0 on
 * invalid sizes. */
size_t kvq_sdpa_decode_workspace_bytes(int B, int Hq, int Hkv, int n_slots, int D);

/* Decode attention (Lq = 1) over quantized K/V caches ([ABADDON]
 * forward_attention; [PR20351] kv_len bound; [PR24473] additive mask for
 * ring/sink caches):
 *   out[b, h, 0, :] = softmax_j(sm_scale * q[b,h,0,:] . k_hat[b,g,j,:] + mask[b,j]) v_hat[b,g,j,:]
 * over j in [0, kv_len), g = h / (Hq / Hkv), k_hat / v_hat dequantized on the
 * fly: (code - zp) * scale for the affine modes (INT8_TH, UINT4_TH),
 * decode(code) * scale of the element's 32-element block for the five block
 * modes (FP8E4M3_B32, FP8E5M2_B32, MXFP8_B32, MXFP4_B32, INT8_B32, MXFP4E1M2_B32: the read
 * side of [IQC]'s per-block write).  A slot at or past kv_len, or one the
 * mask sets to -inf, takes no part at all (its codes and scales may hold any
 * bytes, NaN included).  A row with no visible key gives 0.
 * q: [B, Hq, 1, D] (q_dtype); out: [B, Hq, 1, D] (out_dtype).
 * k, v: caches of one mode (any of the seven) with equal sizes; Hq % heads == 0.
 * kv_len: device int32 scalar or NULL (= n_slots); a value outside
 *   [1, n_slots] is clamped and sets KVQ_FLAG_KVLEN.
 * mask: NULL or fp32 [B, n_slots] with batch stride mask_stride_b (0 shares
 *   one row); values 0 or -inf.  mask_is_causal is accepted for symmetry with
 *   prefill: at Lq = 1 the causal bound is kv_len itself.
 * workspace: device buffer of kvq_sdpa_decode_workspace_bytes() bytes,
 *   16-byte aligned.  Its counter region must be zero when a call starts;
 *   every call leaves it zero, so zero-fill a new workspace once (and again
 *   after writing anything else into it).  The rest holds per-split partial
 *   results and needs no initialisation.  Calls that overlap in time
 *   (different streams) need separate workspaces.
 * Supported D: 64, 128, 256; Hq / heads in {1, 2, 4, 8}. */
kvq_status kvq_sdpa_decode(const void* q, int q_dtype, int B, int Hq,
                           const kvq_cache* k, const kvq_cache* v,
                           const int32_t* kv_len, const float* mask, int64_t mask_stride_b,
                           int mask_is_causal, float sm_scale, void* out, int out_dtype,
                           void* workspace, size_t workspace_bytes,
                           int32_t* err_flags, void* stream);

/* One decode step of a full-context cache in a single launch: the new
 * token's K and V written into the caches, then attention over them
 * ([ABADDON] append followed by forward_attention; [PR20351] commit notes: the
 * new token goes to the cache at the device-side input position, and the key
 * loop stops at the filled length).  Exactly
 *   kvq_quant_scatter_kv_full(xk, xv, x_dtype, B, Hkv, 1, D, x_stride_b,
 *                             x_stride_h, 0, start_pos, k, v, err_flags)
 * followed by kvq_sdpa_decode(q, ..., kv_len = *start_pos + 1, no mask, ...):
 * the same cache bytes and the same output bits, and the same flags (a
 * *start_pos < 0 writes nothing and sets KVQ_FLAG_SLOT_RANGE | KVQ_FLAG_KVLEN
 * with kv_len 1; a *start_pos >= n_slots writes nothing and sets
 * KVQ_FLAG_POS_CAPACITY | KVQ_FLAG_KVLEN with kv_len n_slots).
 * xk, xv: [B, Hkv, 1, D] (x_dtype KVQ_F32 or KVQ_BF16) with element strides
 *   x_stride_b, x_stride_h (>= 0) and unit stride along D; Hkv = k->heads.
 * start_pos: device int32 scalar.  q, out, sm_scale, workspace (the size
 *   kvq_sdpa_decode_workspace_bytes gives, same rules) as kvq_sdpa_decode.
 * Supported: INT8_TH caches whose sizes the single-pass int8 kernel takes
 *   (D 64, 128, 256; Hq / heads in {1, 2, 4, 8}, not 8 at D = 256;
 *   n_slots % 4 == 0; 4-byte aligned zero-point arrays); anything else gives
 *   KVQ_ERR_UNSUPPORTED with nothing enqueued. */
kvq_status kvq_sdpa_decode_append_full(const void* q, int q_dtype, int B, int Hq,
                                       const void* xk, const void* xv, int x_dtype,
                                       int64_t x_stride_b, int64_t x_stride_h, const int32_t* start_pos,
                                       const kvq_cache* k, const kvq_cache* v, float sm_scale,
                                       void* out, int out_dtype, void* workspace, size_t workspace_bytes,
                                       int32_t* err_flags, void* stream);

/* The same one-launch decode step for a sink or ring cache ([PR24473]: the
 * positions manager with sink picks the slot, keys attend through the
 * additive mask built from the slots' positions; a ring cache is sink_size
 * 0).  Exactly
 *   kvq_positions_with_sink(start_pos, 1, sink_size, window, slot,
 *                           cache_positions, err_flags),
 *   kvq_quant_scatter_kv(xk, xv, x_dtype, B, Hkv, 1, D, x_stride_b,
 *                        x_stride_h, 0, slot, 0, k, v, err_flags),
 *   kvq_build_mask(cache_positions, n_slots, start_pos, 1, sink_size,
 *                  window, mask) and
 *   kvq_sdpa_decode(q, ..., kv_len = min(*start_pos + 1, n_slots), mask, ...):
 * the same cache bytes, cache_positions, output bits and flags (a negative
 * *start_pos writes nothing, sets KVQ_FLAG_SLOT_RANGE | KVQ_FLAG_KVLEN and
 * every key is masked: the output is 0).  The mask is never materialized:
 * each key's visibility (cp >= 0, cp <= p and (cp < sink_size or p - cp <
 * window), cp its slot's position) is decided as its tile is read.
 * cache_positions: int32 [n_slots], in/out (-1 = empty).  sink_size >= 0,
 * window >= 1 and sink_size + window == n_slots (else KVQ_ERR_SHAPE).
 * Everything else as kvq_sdpa_decode_append_full. */
kvq_status kvq_sdpa_decode_append_sink(const void* q, int q_dtype, int B, int Hq,
                                       const void* xk, const void* xv, int x_dtype,
                                       int64_t x_stride_b, int64_t x_stride_h, const int32_t* start_pos,
                                       int sink_size, int window, int32_t* cache_positions,
                                       const kvq_cache* k, const kvq_cache* v, float sm_scale,
                                       void* out, int out_dtype, void* workspace, size_t workspace_bytes,
                                       int32_t* err_flags, void* stream);

/* kvq_sdpa_decode with one filled length per batch row: kv_lens is a device
 * int32 array [B] (batch row b attends slots [0, kv_lens[b])), each clamped to
 * [1, n_slots] with KVQ_FLAG_KVLEN.  Otherwise as kvq_sdpa_decode; the same
 * workspace size.  KVQ_ERR_NULL when kv_lens is NULL.  ([PR20351] kv_len
 * bound, applied per sequence of the batch.) */
kvq_status kvq_sdpa_decode_varlen(const void* q, int q_dtype, int B, int Hq,
                                  const kvq_cache* k, const kvq_cache* v,
                                  const int32_t* kv_lens, const float* mask, int64_t mask_stride_b,
                                  float sm_scale, void* out, int out_dtype,
                                  void* workspace, size_t workspace_bytes,
                                  int32_t* err_flags, void* stream);

/* kvq_sdpa_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, arguments and results as kvq_sdpa_decode, without the
 * workspace arguments.  The counters and partials live in one library-owned
 * device array per GPU of KVQ_DECODE_NOALLOC_BYTES bytes (a fixed counter
 * block of KVQ_DECODE_NOALLOC_CTR_BYTES, then the partials), placed with the
 * code object and held until the process ends.  The first call on a device,
 * with that device current, looks up the array's address and enqueues a
 * clear of the counter block on `stream`; no call allocates, frees or calls
 * an allocating routine.  KVQ_ERR_WORKSPACE, with nothing enqueued, when the
 * call needs more: B * heads tickets above the counter block, or partials
 * above the rest (at D = 128, Hq = 32 every shape fits).  Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and give wrong results; order them. */
#define KVQ_DECODE_NOALLOC_BYTES (16u << 20)
#define KVQ_DECODE_NOALLOC_CTR_BYTES (64u << 10)
kvq_status kvq_sdpa_decode_noalloc(const void* q, int q_dtype, int B, int Hq,
                                   const kvq_cache* k, const kvq_cache* v,
                                   const int32_t* kv_len, const float* mask, int64_t mask_stride_b,
                                   int mask_is_causal, float sm_scale, void* out, int out_dtype,
                                   int32_t* err_flags, void* stream);

/* Chunked-prefill attention over quantized K/V caches ([PR20351]): the Lq
 * query rows sit at positions [kv_len - Lq, kv_len); row r attends keys
 * j < kv_len, and when mask_is_causal only j <= kv_len - Lq + r.  The KV loop
 * of a tile of rows stops at the per-tile causal bound
 *   loop_end = min(kv_len, kv_len - Lq + max_row + 1)
 * (flag KVQ_NO_CAUSAL_SKIP scans all tiles below kv_len instead; the result
 * is bit-identical).  mask: NULL or fp32 [Lq, n_slots] shared over the batch
 * (0 / -inf).  q: [B, Hq, Lq, D] (q_dtype); out: [B, Hq, Lq, D] (out_dtype).
 * kv_len: device int32 scalar or NULL (= n_slots), clamped to [Lq, n_slots]
 * with KVQ_FLAG_KVLEN.  Dequantization as in kvq_sdpa_decode.  Supported: any
 * cache mode, D in {64, 128, 256}, Hq / heads in {1, 2, 4, 8}, Lq >= 1. */
kvq_status kvq_sdpa_prefill(const void* q, int q_dtype, int B, int Hq, int Lq,
                            const kvq_cache* k, const kvq_cache* v,
                            const int32_t* kv_len, const float* mask, int mask_is_causal,
                            unsigned flags, float sm_scale, void* out, int out_dtype,
                            int32_t* err_flags, void* stream);

/* kvq_sdpa_prefill with one filled length per batch row: kv_lens is a device
 * int32 array [B]; the Lq query rows of batch row b sit at positions
 * [kv_lens[b] - Lq, kv_lens[b]), each value clamped to [Lq, n_slots] with
 * KVQ_FLAG_KVLEN.  Otherwise as kvq_sdpa_prefill.  KVQ_ERR_NULL when kv_lens
 * is NULL. */
kvq_status kvq_sdpa_prefill_varlen(const void* q, int q_dtype, int B, int Hq, int Lq,
                                   const kvq_cache* k, const kvq_cache* v,
                                   const int32_t* kv_lens, const float* mask, int mask_is_causal,
                                   unsigned flags, float sm_scale, void* out, int out_dtype,
                                   int32_t* err_flags, void* stream);

/* kvq_sdpa_prefill for chunks too short to fill the GPU with query tiles alone
 * (the chunked prefill of [PR20351] with a small Lq, which gives
 * B * heads * ceil(Lq * (Hq / heads) / 128) workgroups): each query tile's
 * key range, below its per-tile causal bound, is split over several
 * workgroups, and the splits' partial (max, sum, output) are merged per query
 * row afterwards, as in decode.  Arguments, bounds, masks, errors and result
 * as kvq_sdpa_prefill, within the same tolerance (the split changes the
 * summation order, so the bits may differ from it; KVQ_NO_CAUSAL_SKIP is
 * bit-identical to the default here too), plus:
 * workspace: device buffer, 16-byte aligned, of at least
 *   kvq_sdpa_prefill_split_workspace_bytes(B, Hq, heads, Lq, n_slots, D)
 *   bytes ([B*Hq*Lq, splits, D + 2] fp32 partials; no initialisation needed;
 *   calls that overlap in time need separate workspaces).  KVQ_ERR_WORKSPACE
 *   when it is missing, misaligned or too small.  A size of 0 means the query
 *   tiles fill the part already: the call then runs as kvq_sdpa_prefill and
 *   workspace may be NULL.  The split count depends on the sizes only (about
 *   256 workgroups, at least 256 keys of n_slots per split, at most 64). */
size_t kvq_sdpa_prefill_split_workspace_bytes(int B, int Hq, int heads, int Lq, int n_slots, int D);
kvq_status kvq_sdpa_prefill_split(const void* q, int q_dtype, int B, int Hq, int Lq,
                                  const kvq_cache* k, const kvq_cache* v,
                                  const int32_t* kv_len, const float* mask, int mask_is_causal,
                                  unsigned flags, float sm_scale, void* out, int out_dtype,
                                  void* workspace, size_t workspace_bytes,
                                  int32_t* err_flags, void* stream);

/* kvq_sdpa_prefill_split with one filled length per batch row, as
 * kvq_sdpa_prefill_varlen ([PR20351] kv_len bound per sequence): kv_lens is a
 * device int32 array [B], each value clamped to [Lq, n_slots] with
 * KVQ_FLAG_KVLEN; the same workspace size.  KVQ_ERR_NULL when kv_lens is NULL. */
kvq_status kvq_sdpa_prefill_split_varlen(const void* q, int q_dtype, int B, int Hq, int Lq,
                                         const kvq_cache* k, const kvq_cache* v,
                                         const int32_t* kv_lens, const float* mask, int mask_is_causal,
                                         unsigned flags, float sm_scale, void* out, int out_dtype,
                                         void* workspace, size_t workspace_bytes,
                                         int32_t* err_flags, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
