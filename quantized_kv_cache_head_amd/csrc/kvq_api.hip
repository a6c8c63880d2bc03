// kvq_api.hip -- the C ABI of libkvq: argument validation, sizes, launches.
//
// Every entry point validates on the host and returns a kvq_status without
// enqueuing anything when an argument is rejected; otherwise it enqueues on
// the caller's stream and returns without synchronizing.  The library never
// allocates device memory; the one device array it owns is the fixed-size
// scratch of kvq_sdpa_decode_noalloc, placed with the code object.
// Unsupported-but-valid requests are rejected with KVQ_ERR_UNSUPPORTED rather
// than run in a degraded form (pytorch/executorch
// PR 24473, Summary: caches that cannot be run are rejected, never flattened).
#include "../../include/kvq.h"
#include "kvq_internal.h"

#include <mutex>

#define KVQ_API extern "C" __attribute__((visibility("default")))

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int row_bytes(int qmode, int D) {
    return (qmode == KVQ_UINT4_TH || qmode == KVQ_MXFP4_B32 || qmode == KVQ_MXFP4E1M2_B32) ? D / 2 : D;
}
bool is_affine(int qmode) { return qmode == KVQ_INT8_TH || qmode == KVQ_UINT4_TH; }
bool is_mx(int qmode) { return qmode == KVQ_MXFP4_B32 || qmode == KVQ_MXFP8_B32 || qmode == KVQ_MXFP4E1M2_B32; }
int scales_per_row(int qmode, int D) { return is_affine(qmode) ? 1 : D / 32; }
int scale_bytes(int qmode) { return is_mx(qmode) ? 1 : 4; }

kvq_status check_dims(int qmode, int D) {
    if (qmode < KVQ_INT8_TH || qmode > KVQ_MXFP4E1M2_B32) return KVQ_ERR_DTYPE;
    if (D <= 0 || D > 8192) return KVQ_ERR_SHAPE;
    if (is_affine(qmode) ? (D % 8 != 0) : (D % 32 != 0)) return KVQ_ERR_SHAPE;
    return KVQ_OK;
}

kvq_status check_cache(const kvq_cache* c) {
    if (!c) return KVQ_ERR_NULL;
    kvq_status st = check_dims(c->qmode, c->head_dim);
    if (st != KVQ_OK) return st;
    if (c->batch <= 0 || c->heads <= 0 || c->n_slots <= 0) return KVQ_ERR_SHAPE;
    if (!c->codes || !c->scales) return KVQ_ERR_NULL;
    if (is_affine(c->qmode) && !c->zps) return KVQ_ERR_NULL;
    // code rows are written and read 4..16 bytes at a time
    if (!aligned(c->codes, 16) || !aligned(c->scales, 4)) return KVQ_ERR_SHAPE;
    return KVQ_OK;
}

kvq_status from_hip(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH; }

// The scatter kernels index lanes (8 elements each) in 32 bits.
bool scatter_size_ok(int B, int H, int T, int D) { return (int64_t)B * H * T * (D / 8) < (int64_t(1) << 31); }

}  // namespace

KVQ_API const char* kvq_status_string(kvq_status s) {
    switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "null pointer argument";
    case KVQ_ERR_SHAPE: return "size, stride or alignment out of the supported range";
    case KVQ_ERR_DTYPE: return "dtype or quantization mode not valid for this call";
    case KVQ_ERR_UNSUPPORTED: return "configuration not supported by this build";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

KVQ_API kvq_status kvq_cache_bytes(int qmode, int B, int H, int n_slots, int D, size_t* codes_bytes,
                                   size_t* scales_bytes, size_t* zps_bytes) {
    kvq_status st = check_dims(qmode, D);
    if (st != KVQ_OK) return st;
    if (B <= 0 || H <= 0 || n_slots <= 0) return KVQ_ERR_SHAPE;
    const size_t rows = (size_t)B * H * n_slots;
    if (codes_bytes) *codes_bytes = rows * row_bytes(qmode, D);
    if (scales_bytes) *scales_bytes = rows * scales_per_row(qmode, D) * scale_bytes(qmode);
    if (zps_bytes) *zps_bytes = is_affine(qmode) ? rows : 0;
    return KVQ_OK;
}

KVQ_API kvq_status kvq_quant_scatter_flags(const void* x, int x_dtype, int B, int H, int T, int D,
                                           int64_t stride_b, int64_t stride_h, int64_t stride_t,
                                           const int32_t* slot_mapping, int64_t slot_stride_b,
                                           const kvq_cache* cache, unsigned flags, int32_t* err_flags,
                                           void* stream) {
    kvq_status st = check_cache(cache);
    if (st != KVQ_OK) return st;
    if ((flags & ~KVQ_MX_SCALE_OCP) || ((flags & KVQ_MX_SCALE_OCP) && !is_mx(cache->qmode)))
        return KVQ_ERR_UNSUPPORTED;
    if (x_dtype != KVQ_F32 && x_dtype != KVQ_BF16) return KVQ_ERR_DTYPE;
    if (T < 0 || B != cache->batch || H != cache->heads || D != cache->head_dim) return KVQ_ERR_SHAPE;
    if (T == 0) return KVQ_OK;
    if (!x || !slot_mapping) return KVQ_ERR_NULL;
    if (stride_b < 0 || stride_h < 0 || stride_t < 0 || slot_stride_b < 0) return KVQ_ERR_SHAPE;
    // 8 elements per lane are loaded with 16-byte loads
    const int64_t vec = x_dtype == KVQ_BF16 ? 8 : 4;
    if (!aligned(x, 16) || stride_b % vec || stride_h % vec || stride_t % vec) return KVQ_ERR_SHAPE;
    if (!scatter_size_ok(B, H, T, D)) return KVQ_ERR_SHAPE;
    return from_hip(kvq::launch_quant_scatter(cache->qmode, x_dtype == KVQ_BF16, x, B, H, T, D, stride_b, stride_h,
                                              stride_t, slot_mapping, slot_stride_b, cache->n_slots,
                                              reinterpret_cast<uint8_t*>(cache->codes), cache->scales, cache->zps,
                                              (int)flags, err_flags, reinterpret_cast<hipStream_t>(stream)));
}

KVQ_API kvq_status kvq_quant_scatter(const void* x, int x_dtype, int B, int H, int T, int D, int64_t stride_b,
                                     int64_t stride_h, int64_t stride_t, const int32_t* slot_mapping,
                                     int64_t slot_stride_b, const kvq_cache* cache, int32_t* err_flags,
                                     void* stream) {
    return kvq_quant_scatter_flags(x, x_dtype, B, H, T, D, stride_b, stride_h, stride_t, slot_mapping,
                                   slot_stride_b, cache, 0u, err_flags, stream);
}

// K and V caches of one update: same mode and sizes, x as the scatter takes it.
static kvq_status check_kv_update(const void* xk, const void* xv, int x_dtype, int B, int H, int T, int D,
                                  int64_t stride_b, int64_t stride_h, int64_t stride_t, const kvq_cache* k_cache,
                                  const kvq_cache* v_cache) {
    kvq_status st = check_cache(k_cache);
    if (st != KVQ_OK) return st;
    if ((st = check_cache(v_cache)) != KVQ_OK) return st;
    if (k_cache->qmode != v_cache->qmode || k_cache->batch != v_cache->batch || k_cache->heads != v_cache->heads ||
        k_cache->n_slots != v_cache->n_slots || k_cache->head_dim != v_cache->head_dim)
        return KVQ_ERR_SHAPE;
    if (x_dtype != KVQ_F32 && x_dtype != KVQ_BF16) return KVQ_ERR_DTYPE;
    if (T < 0 || B != k_cache->batch || H != k_cache->heads || D != k_cache->head_dim) return KVQ_ERR_SHAPE;
    if (T == 0) return KVQ_OK;
    if (!xk || !xv) return KVQ_ERR_NULL;
    if (stride_b < 0 || stride_h < 0 || stride_t < 0) return KVQ_ERR_SHAPE;
    const int64_t vec = x_dtype == KVQ_BF16 ? 8 : 4;
    if (!aligned(xk, 16) || !aligned(xv, 16) || stride_b % vec || stride_h % vec || stride_t % vec)
        return KVQ_ERR_SHAPE;
    if (!scatter_size_ok(B, H, T, D)) return KVQ_ERR_SHAPE;
    return KVQ_OK;
}

KVQ_API kvq_status kvq_quant_scatter_kv(const void* xk, const void* xv, int x_dtype, int B, int H, int T, int D,
                                        int64_t stride_b, int64_t stride_h, int64_t stride_t,
                                        const int32_t* slot_mapping, int64_t slot_stride_b, const kvq_cache* k_cache,
                                        const kvq_cache* v_cache, int32_t* err_flags, void* stream) {
    const kvq_status st = check_kv_update(xk, xv, x_dtype, B, H, T, D, stride_b, stride_h, stride_t, k_cache, v_cache);
    if (st != KVQ_OK || T == 0) return st;
    if (!slot_mapping) return KVQ_ERR_NULL;
    if (slot_stride_b < 0) return KVQ_ERR_SHAPE;
    return from_hip(kvq::launch_quant_scatter_kv(
        k_cache->qmode, x_dtype == KVQ_BF16, xk, xv, B, H, T, D, stride_b, stride_h, stride_t, slot_mapping,
        slot_stride_b, k_cache->n_slots, reinterpret_cast<uint8_t*>(k_cache->codes), k_cache->scales, k_cache->zps,
        reinterpret_cast<uint8_t*>(v_cache->codes), v_cache->scales, v_cache->zps, nullptr, err_flags,
        reinterpret_cast<hipStream_t>(stream)));
}

KVQ_API kvq_status kvq_quant_scatter_kv_full(const void* xk, const void* xv, int x_dtype, int B, int H, int T, int D,
                                             int64_t stride_b, int64_t stride_h, int64_t stride_t,
                                             const int32_t* start_pos, const kvq_cache* k_cache,
                                             const kvq_cache* v_cache, int32_t* err_flags, void* stream) {
    const kvq_status st = check_kv_update(xk, xv, x_dtype, B, H, T, D, stride_b, stride_h, stride_t, k_cache, v_cache);
    if (st != KVQ_OK || T == 0) return st;
    if (!start_pos) return KVQ_ERR_NULL;
    return from_hip(kvq::launch_quant_scatter_kv(
        k_cache->qmode, x_dtype == KVQ_BF16, xk, xv, B, H, T, D, stride_b, stride_h, stride_t, nullptr, 0,
        k_cache->n_slots, reinterpret_cast<uint8_t*>(k_cache->codes), k_cache->scales, k_cache->zps,
        reinterpret_cast<uint8_t*>(v_cache->codes), v_cache->scales, v_cache->zps, start_pos, err_flags,
        reinterpret_cast<hipStream_t>(stream)));
}

KVQ_API kvq_status kvq_positions_with_sink(const int32_t* start_pos, int T, int sink_size, int window,
                                           int32_t* slot_mapping_out, int32_t* cache_positions,
                                           int32_t* err_flags, void* stream) {
    if (T < 0 || sink_size < 0 || window < 1 || (int64_t)sink_size + window > INT32_MAX) return KVQ_ERR_SHAPE;
    if (T == 0) return KVQ_OK;
    if (!start_pos || !slot_mapping_out) return KVQ_ERR_NULL;
    return from_hip(kvq::launch_positions_sink(start_pos, T, sink_size, window, slot_mapping_out, cache_positions,
                                               err_flags, reinterpret_cast<hipStream_t>(stream)));
}

KVQ_API kvq_status kvq_positions_ring(const int32_t* start_pos, int T, int window, int32_t* slot_mapping_out,
                                      int32_t* cache_positions, int32_t* err_flags, void* stream) {
    return kvq_positions_with_sink(start_pos, T, 0, window, slot_mapping_out, cache_positions, err_flags, stream);
}

KVQ_API kvq_status kvq_positions_full(const int32_t* start_pos, int T, int capacity, int32_t* slot_mapping_out,
                                      int32_t* cache_positions, int32_t* err_flags, void* stream) {
    if (T < 0 || capacity < 1) return KVQ_ERR_SHAPE;
    if (T == 0) return KVQ_OK;
    if (!start_pos || !slot_mapping_out) return KVQ_ERR_NULL;
    return from_hip(kvq::launch_positions_full(start_pos, T, capacity, slot_mapping_out, cache_positions, err_flags,
                                               reinterpret_cast<hipStream_t>(stream)));
}

KVQ_API kvq_status kvq_build_mask(const int32_t* cache_positions, int n_slots, const int32_t* start_pos, int Lq,
                                  int sink_size, int window, float* mask_out, void* stream) {
    if (n_slots < 1 || Lq < 0 || sink_size < 0 || window < 1) return KVQ_ERR_SHAPE;
    // the cache holds the sink slots and the window, nothing else
    if ((int64_t)sink_size + window != n_slots) return KVQ_ERR_SHAPE;
    if (Lq == 0) return KVQ_OK;
    if (!cache_positions || !start_pos || !mask_out) return KVQ_ERR_NULL;
    return from_hip(kvq::launch_build_mask(cache_positions, n_slots, start_pos, Lq, sink_size, window, mask_out,
                                           reinterpret_cast<hipStream_t>(stream)));
}

namespace {

kvq_status check_attention(const void* q, int q_dtype, int B, int Hq, const kvq_cache* k, const kvq_cache* v,
                           void* out, int out_dtype) {
    kvq_status st = check_cache(k);
    if (st != KVQ_OK) return st;
    st = check_cache(v);
    if (st != KVQ_OK) return st;
    if (!q || !out) return KVQ_ERR_NULL;
    if ((q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) || (out_dtype != KVQ_F32 && out_dtype != KVQ_BF16))
        return KVQ_ERR_DTYPE;
    if (k->qmode != v->qmode) return KVQ_ERR_DTYPE;
    if (k->batch != v->batch || k->heads != v->heads || k->n_slots != v->n_slots || k->head_dim != v->head_dim)
        return KVQ_ERR_SHAPE;
    if (B != k->batch || Hq <= 0 || Hq % k->heads != 0) return KVQ_ERR_SHAPE;
    const int G = Hq / k->heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return KVQ_ERR_UNSUPPORTED;
    const int D = k->head_dim;
    if (D != 64 && D != 128 && D != 256) return KVQ_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(out, 4)) return KVQ_ERR_SHAPE;
    return KVQ_OK;
}

// Decode workspace: a counter region (one ticket per (b, kv head), which the
// single-pass kernel needs at zero when a call starts and leaves at zero),
// then the per-split partials, fp32: (m, l) and o for every (b, kv head,
// split, query head of the group).
size_t decode_ctr_bytes(int B, int Hkv) { return ((size_t)B * Hkv * sizeof(unsigned) + 255) / 256 * 256; }

size_t decode_part_bytes(int B, int Hq, int splits, int D) {
    return (size_t)B * Hq * splits * ((size_t)D + 2) * sizeof(float);
}

int decode_splits_any(int B, int Hq, int Hkv, int S, int D) {
    const int a = kvq::decode_splits_max(B, Hq, Hkv, S, D, KVQ_INT8_TH);
    const int b = kvq::decode_splits_max(B, Hq, Hkv, S, D, KVQ_UINT4_TH);
    return a > b ? a : b;
}

}  // namespace

KVQ_API size_t kvq_sdpa_decode_workspace_bytes(int B, int Hq, int Hkv, int n_slots, int D) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_slots <= 0 || D <= 0 || D % 16 || Hq % Hkv) return 0;
    size_t part = decode_part_bytes(B, Hq, decode_splits_any(B, Hq, Hkv, n_slots, D), D);
    const int G = Hq / Hkv;
    if (kvq::mfma_supported(KVQ_INT8_TH, D, G, n_slots)) {
        const size_t ps = decode_part_bytes(B, Hq, kvq::mfma_splits_max(B, Hkv, n_slots, D, G), D);
        if (ps > part) part = ps;
    }
    return decode_ctr_bytes(B, Hkv) + part;
}

namespace {

// Split count and partial bytes of one decode call: the single-pass int8
// kernel where it applies (its ticket counters live in the counter region),
// else the split pass plus combine kernel.
struct DecodePlan {
    bool single;
    int nsplit;
    size_t part_bytes;
};

DecodePlan decode_plan(int q_dtype, int B, int Hq, const kvq_cache* k, const kvq_cache* v) {
    const int D = k->head_dim;
    const int G = Hq / k->heads;
    DecodePlan p;
    p.single = kvq::mfma_supported(k->qmode, D, G, k->n_slots) && aligned(k->zps, 4) && aligned(v->zps, 4);
    p.nsplit = p.single ? kvq::mfma_splits(B, k->heads, k->n_slots, D, G, q_dtype == KVQ_BF16)
                        : kvq::decode_splits(B, Hq, k->heads, k->n_slots, D, k->qmode, q_dtype == KVQ_BF16);
    p.part_bytes = decode_part_bytes(B, Hq, p.nsplit, D);
    return p;
}

// Enqueue a validated decode call: ctr holds one zero ticket per (b, kv
// head), part at least plan.part_bytes bytes (16-byte aligned).
kvq_status sdpa_decode_enqueue(const DecodePlan& plan, const void* q, int q_dtype, int B, int Hq,
                               const kvq_cache* k, const kvq_cache* v, const int32_t* kv_len, int kv_len_sb,
                               const float* mask, int64_t mask_stride_b, float sm_scale, void* out, int out_dtype,
                               unsigned* ctr, float* part, int32_t* err_flags, void* stream) {
    kvq::DecodeLaunch L;
    L.q = q;
    L.q_bf16 = q_dtype == KVQ_BF16;
    L.B = B;
    L.Hq = Hq;
    L.Hkv = k->heads;
    L.S = k->n_slots;
    L.D = k->head_dim;
    L.qmode = k->qmode;
    L.kc = reinterpret_cast<const uint8_t*>(k->codes);
    L.ks = reinterpret_cast<const float*>(k->scales);
    L.kz = k->zps;
    L.vc = reinterpret_cast<const uint8_t*>(v->codes);
    L.vs = reinterpret_cast<const float*>(v->scales);
    L.vz = v->zps;
    L.kv_len = kv_len;
    L.kv_len_sb = kv_len_sb;
    L.mask = mask;
    L.mask_sb = mask_stride_b;
    L.sm_scale = sm_scale;
    L.out = out;
    L.out_bf16 = out_dtype == KVQ_BF16;
    L.nsplit = plan.nsplit;
    L.err = err_flags;
    L.ctr = ctr;
    if (plan.single) {
        L.part_ml = part;
        L.part_o = part + (size_t)B * Hq * plan.nsplit * 2;
        return from_hip(kvq::launch_sdpa_decode_mfma(L, reinterpret_cast<hipStream_t>(stream)));
    }
    L.part_o = part;
    L.part_ml = L.part_o + (size_t)B * Hq * plan.nsplit * L.D;
    return from_hip(kvq::launch_sdpa_decode(L, reinterpret_cast<hipStream_t>(stream)));
}

kvq_status sdpa_decode_impl(const void* q, int q_dtype, int B, int Hq, const kvq_cache* k, const kvq_cache* v,
                            const int32_t* kv_len, int kv_len_sb, const float* mask, int64_t mask_stride_b,
                            float sm_scale, void* out, int out_dtype, void* workspace, size_t workspace_bytes,
                            int32_t* err_flags, void* stream) {
    kvq_status st = check_attention(q, q_dtype, B, Hq, k, v, out, out_dtype);
    if (st != KVQ_OK) return st;
    if (mask_stride_b < 0) return KVQ_ERR_SHAPE;
    const DecodePlan plan = decode_plan(q_dtype, B, Hq, k, v);
    const size_t ctr = decode_ctr_bytes(B, k->heads);
    if (!workspace || workspace_bytes < ctr + plan.part_bytes || !aligned(workspace, 16)) return KVQ_ERR_WORKSPACE;
    return sdpa_decode_enqueue(plan, q, q_dtype, B, Hq, k, v, kv_len, kv_len_sb, mask, mask_stride_b, sm_scale,
                               out, out_dtype, reinterpret_cast<unsigned*>(workspace),
                               reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + ctr), err_flags, stream);
}

// Bytes of a key-split prefill's partials: [B * Hq * Lq, splits, D + 2] fp32.
size_t prefill_ws_bytes(int splits, int B, int Hq, int Lq, int D) {
    return splits > 1 ? (size_t)B * Hq * Lq * splits * ((size_t)D + 2) * sizeof(float) : 0;
}

kvq_status sdpa_prefill_impl(const void* q, int q_dtype, int B, int Hq, int Lq, const kvq_cache* k,
                             const kvq_cache* v, const int32_t* kv_len, int kv_len_sb, const float* mask,
                             int mask_is_causal, unsigned flags, float sm_scale, void* out, int out_dtype,
                             bool split, void* workspace, size_t workspace_bytes, int32_t* err_flags,
                             void* stream) {
    kvq_status st = check_attention(q, q_dtype, B, Hq, k, v, out, out_dtype);
    if (st != KVQ_OK) return st;
    if (Lq < 1 || Lq > k->n_slots) return KVQ_ERR_SHAPE;
    if (flags & ~KVQ_NO_CAUSAL_SKIP) return KVQ_ERR_UNSUPPORTED;
    const int splits = split ? kvq::prefill_kv_splits(B, Hq, k->heads, Lq, k->n_slots) : 1;
    const size_t need = prefill_ws_bytes(splits, B, Hq, Lq, k->head_dim);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16))) return KVQ_ERR_WORKSPACE;
    kvq::PrefillLaunch L;
    L.q = q;
    L.q_bf16 = q_dtype == KVQ_BF16;
    L.B = B;
    L.Hq = Hq;
    L.Hkv = k->heads;
    L.S = k->n_slots;
    L.D = k->head_dim;
    L.Lq = Lq;
    L.qmode = k->qmode;
    L.kc = reinterpret_cast<const uint8_t*>(k->codes);
    L.ks = reinterpret_cast<const float*>(k->scales);
    L.kz = k->zps;
    L.vc = reinterpret_cast<const uint8_t*>(v->codes);
    L.vs = reinterpret_cast<const float*>(v->scales);
    L.vz = v->zps;
    L.kv_len = kv_len;
    L.kv_len_sb = kv_len_sb;
    L.mask = mask;
    L.causal = mask_is_causal != 0;
    L.no_skip = (flags & KVQ_NO_CAUSAL_SKIP) != 0;
    L.sm_scale = sm_scale;
    L.out = out;
    L.out_bf16 = out_dtype == KVQ_BF16;
    L.err = err_flags;
    L.kv_splits = splits;
    if (splits > 1) {
        L.part_o = reinterpret_cast<float*>(workspace);
        L.part_ml = L.part_o + (size_t)B * Hq * Lq * splits * k->head_dim;
    }
    hipError_t e = kvq::launch_sdpa_prefill(L, reinterpret_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return KVQ_ERR_UNSUPPORTED;
    return from_hip(e);
}

}  // namespace

KVQ_API kvq_status kvq_sdpa_decode(const void* q, int q_dtype, int B, int Hq, const kvq_cache* k,
                                   const kvq_cache* v, const int32_t* kv_len, const float* mask,
                                   int64_t mask_stride_b, int mask_is_causal, float sm_scale, void* out,
                                   int out_dtype, void* workspace, size_t workspace_bytes, int32_t* err_flags,
                                   void* stream) {
    (void)mask_is_causal;   // at Lq = 1 the causal bound equals kv_len
    return sdpa_decode_impl(q, q_dtype, B, Hq, k, v, kv_len, 0, mask, mask_stride_b, sm_scale, out, out_dtype,
                            workspace, workspace_bytes, err_flags, stream);
}

namespace {

// The one-launch decode step (append variant of the single-pass int8
// kernel); cpos NULL: full-context layout, else sink / ring.
kvq_status sdpa_decode_append_impl(const void* q, int q_dtype, int B, int Hq, const void* xk, const void* xv,
                                   int x_dtype, int64_t x_stride_b, int64_t x_stride_h, const int32_t* start_pos,
                                   int32_t* cpos, int sink_size, int window, const kvq_cache* k,
                                   const kvq_cache* v, float sm_scale, void* out, int out_dtype, void* workspace,
                                   size_t workspace_bytes, int32_t* err_flags, void* stream) {
    kvq_status st = check_attention(q, q_dtype, B, Hq, k, v, out, out_dtype);
    if (st != KVQ_OK) return st;
    if (!xk || !xv || !start_pos) return KVQ_ERR_NULL;
    if (x_dtype != KVQ_F32 && x_dtype != KVQ_BF16) return KVQ_ERR_DTYPE;
    if (x_stride_b < 0 || x_stride_h < 0) return KVQ_ERR_SHAPE;
    const size_t es = x_dtype == KVQ_BF16 ? 2 : 4;
    if (!aligned(xk, es) || !aligned(xv, es)) return KVQ_ERR_SHAPE;
    if (cpos && !aligned(cpos, 4)) return KVQ_ERR_SHAPE;
    const DecodePlan plan = decode_plan(q_dtype, B, Hq, k, v);
    if (!plan.single) return KVQ_ERR_UNSUPPORTED;
    const size_t ctr = decode_ctr_bytes(B, k->heads);
    if (!workspace || workspace_bytes < ctr + plan.part_bytes || !aligned(workspace, 16)) return KVQ_ERR_WORKSPACE;
    kvq::DecodeLaunch L;
    L.q = q;
    L.q_bf16 = q_dtype == KVQ_BF16;
    L.B = B;
    L.Hq = Hq;
    L.Hkv = k->heads;
    L.S = k->n_slots;
    L.D = k->head_dim;
    L.qmode = k->qmode;
    L.kc = reinterpret_cast<const uint8_t*>(k->codes);
    L.ks = reinterpret_cast<const float*>(k->scales);
    L.kz = k->zps;
    L.vc = reinterpret_cast<const uint8_t*>(v->codes);
    L.vs = reinterpret_cast<const float*>(v->scales);
    L.vz = v->zps;
    L.kv_len = nullptr;
    L.kv_len_sb = 0;
    L.mask = nullptr;
    L.mask_sb = 0;
    L.sm_scale = sm_scale;
    L.out = out;
    L.out_bf16 = out_dtype == KVQ_BF16;
    L.nsplit = plan.nsplit;
    L.err = err_flags;
    L.ctr = reinterpret_cast<unsigned*>(workspace);
    float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + ctr);
    L.part_ml = part;
    L.part_o = part + (size_t)B * Hq * plan.nsplit * 2;
    L.start_pos = start_pos;
    L.xk = xk;
    L.xv = xv;
    L.x_bf16 = x_dtype == KVQ_BF16;
    L.xsb = x_stride_b;
    L.xsh = x_stride_h;
    L.cpos = cpos;
    L.sink = sink_size;
    L.window = window;
    return from_hip(kvq::launch_sdpa_decode_mfma(L, reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

KVQ_API kvq_status kvq_sdpa_decode_append_full(const void* q, int q_dtype, int B, int Hq, const void* xk,
                                               const void* xv, int x_dtype, int64_t x_stride_b,
                                               int64_t x_stride_h, const int32_t* start_pos, const kvq_cache* k,
                                               const kvq_cache* v, float sm_scale, void* out, int out_dtype,
                                               void* workspace, size_t workspace_bytes, int32_t* err_flags,
                                               void* stream) {
    return sdpa_decode_append_impl(q, q_dtype, B, Hq, xk, xv, x_dtype, x_stride_b, x_stride_h, start_pos, nullptr, 0,
                                   0, k, v, sm_scale, out, out_dtype, workspace, workspace_bytes, err_flags, stream);
}

KVQ_API kvq_status kvq_sdpa_decode_append_sink(const void* q, int q_dtype, int B, int Hq, const void* xk,
                                               const void* xv, int x_dtype, int64_t x_stride_b,
                                               int64_t x_stride_h, const int32_t* start_pos, int sink_size,
                                               int window, int32_t* cache_positions, const kvq_cache* k,
                                               const kvq_cache* v, float sm_scale, void* out, int out_dtype,
                                               void* workspace, size_t workspace_bytes, int32_t* err_flags,
                                               void* stream) {
    if (!cache_positions) return KVQ_ERR_NULL;
    if (!k) return KVQ_ERR_NULL;
    if (sink_size < 0 || window < 1 || (int64_t)sink_size + window != k->n_slots) return KVQ_ERR_SHAPE;
    return sdpa_decode_append_impl(q, q_dtype, B, Hq, xk, xv, x_dtype, x_stride_b, x_stride_h, start_pos,
                                   cache_positions, sink_size, window, k, v, sm_scale, out, out_dtype, workspace,
                                   workspace_bytes, err_flags, stream);
}

KVQ_API kvq_status kvq_sdpa_decode_varlen(const void* q, int q_dtype, int B, int Hq, const kvq_cache* k,
                                          const kvq_cache* v, const int32_t* kv_lens, const float* mask,
                                          int64_t mask_stride_b, float sm_scale, void* out, int out_dtype,
                                          void* workspace, size_t workspace_bytes, int32_t* err_flags,
                                          void* stream) {
    if (!kv_lens) return KVQ_ERR_NULL;
    return sdpa_decode_impl(q, q_dtype, B, Hq, k, v, kv_lens, 1, mask, mask_stride_b, sm_scale, out, out_dtype,
                            workspace, workspace_bytes, err_flags, stream);
}

// ---- decode without a caller workspace --------------------------------------
// One array per GPU, placed with the code object and held until the process
// ends: a fixed block of ticket counters, then the partials.  The counter
// block has a fixed size and offset, so partial bytes of a call of one shape
// never land where a later call of another shape expects zero tickets.
static __device__ __align__(256) unsigned char scratch[KVQ_DECODE_NOALLOC_BYTES];

namespace {

constexpr size_t kScratchCtrBytes = KVQ_DECODE_NOALLOC_CTR_BYTES;
constexpr size_t kScratchPartBytes = KVQ_DECODE_NOALLOC_BYTES - KVQ_DECODE_NOALLOC_CTR_BYTES;
constexpr int kMaxDevices = 64;
static_assert(kScratchCtrBytes % 256 == 0 && kScratchPartBytes > 0, "scratch layout");

__global__ void zero_words(unsigned* p, unsigned n) {
    for (unsigned i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array.  The first call on a
// device looks it up (the array's host-side name is no device address) and
// clears the counter block on the caller's stream; every decode launch
// leaves its tickets at zero again.
kvq_status device_scratch(hipStream_t stream, char** base) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVQ_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KVQ_ERR_LAUNCH;
        hipLaunchKernelGGL(zero_words, dim3(16), dim3(256), 0, stream, reinterpret_cast<unsigned*>(ptr),
                           static_cast<unsigned>(kScratchCtrBytes / sizeof(unsigned)));
        if (hipGetLastError() != hipSuccess) return KVQ_ERR_LAUNCH;
        g_scratch[dev] = ptr;
    }
    *base = static_cast<char*>(g_scratch[dev]);
    return KVQ_OK;
}

}  // namespace

KVQ_API kvq_status kvq_sdpa_decode_noalloc(const void* q, int q_dtype, int B, int Hq, const kvq_cache* k,
                                           const kvq_cache* v, const int32_t* kv_len, const float* mask,
                                           int64_t mask_stride_b, int mask_is_causal, float sm_scale, void* out,
                                           int out_dtype, int32_t* err_flags, void* stream) {
    (void)mask_is_causal;
    kvq_status st = check_attention(q, q_dtype, B, Hq, k, v, out, out_dtype);
    if (st != KVQ_OK) return st;
    if (mask_stride_b < 0) return KVQ_ERR_SHAPE;
    if ((size_t)B * k->heads * sizeof(unsigned) > kScratchCtrBytes) return KVQ_ERR_WORKSPACE;
    const DecodePlan plan = decode_plan(q_dtype, B, Hq, k, v);
    if (plan.part_bytes > kScratchPartBytes) return KVQ_ERR_WORKSPACE;
    char* base = nullptr;
    st = device_scratch(reinterpret_cast<hipStream_t>(stream), &base);
    if (st != KVQ_OK) return st;
    return sdpa_decode_enqueue(plan, q, q_dtype, B, Hq, k, v, kv_len, 0, mask, mask_stride_b, sm_scale, out,
                               out_dtype, reinterpret_cast<unsigned*>(base),
                               reinterpret_cast<float*>(base + kScratchCtrBytes), err_flags, stream);
}

KVQ_API kvq_status kvq_sdpa_prefill(const void* q, int q_dtype, int B, int Hq, int Lq, const kvq_cache* k,
                                    const kvq_cache* v, const int32_t* kv_len, const float* mask,
                                    int mask_is_causal, unsigned flags, float sm_scale, void* out, int out_dtype,
                                    int32_t* err_flags, void* stream) {
    return sdpa_prefill_impl(q, q_dtype, B, Hq, Lq, k, v, kv_len, 0, mask, mask_is_causal, flags, sm_scale, out,
                             out_dtype, false, nullptr, 0, err_flags, stream);
}

KVQ_API kvq_status kvq_sdpa_prefill_varlen(const void* q, int q_dtype, int B, int Hq, int Lq, const kvq_cache* k,
                                           const kvq_cache* v, const int32_t* kv_lens, const float* mask,
                                           int mask_is_causal, unsigned flags, float sm_scale, void* out,
                                           int out_dtype, int32_t* err_flags, void* stream) {
    if (!kv_lens) return KVQ_ERR_NULL;
    return sdpa_prefill_impl(q, q_dtype, B, Hq, Lq, k, v, kv_lens, 1, mask, mask_is_causal, flags, sm_scale, out,
                             out_dtype, false, nullptr, 0, err_flags, stream);
}

KVQ_API size_t kvq_sdpa_prefill_split_workspace_bytes(int B, int Hq, int Hkv, int Lq, int n_slots, int D) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || Lq <= 0 || n_slots <= 0 || D <= 0) return 0;
    return prefill_ws_bytes(kvq::prefill_kv_splits(B, Hq, Hkv, Lq, n_slots), B, Hq, Lq, D);
}

KVQ_API kvq_status kvq_sdpa_prefill_split(const void* q, int q_dtype, int B, int Hq, int Lq, const kvq_cache* k,
                                          const kvq_cache* v, const int32_t* kv_len, const float* mask,
                                          int mask_is_causal, unsigned flags, float sm_scale, void* out,
                                          int out_dtype, void* workspace, size_t workspace_bytes,
                                          int32_t* err_flags, void* stream) {
    return sdpa_prefill_impl(q, q_dtype, B, Hq, Lq, k, v, kv_len, 0, mask, mask_is_causal, flags, sm_scale, out,
                             out_dtype, true, workspace, workspace_bytes, err_flags, stream);
}

KVQ_API kvq_status kvq_sdpa_prefill_split_varlen(const void* q, int q_dtype, int B, int Hq, int Lq,
                                                 const kvq_cache* k, const kvq_cache* v, const int32_t* kv_lens,
                                                 const float* mask, int mask_is_causal, unsigned flags,
                                                 float sm_scale, void* out, int out_dtype, void* workspace,
                                                 size_t workspace_bytes, int32_t* err_flags, void* stream) {
    if (!kv_lens) return KVQ_ERR_NULL;
    return sdpa_prefill_impl(q, q_dtype, B, Hq, Lq, k, v, kv_lens, 1, mask, mask_is_causal, flags, sm_scale, out,
                             out_dtype, true, workspace, workspace_bytes, err_flags, stream);
}
