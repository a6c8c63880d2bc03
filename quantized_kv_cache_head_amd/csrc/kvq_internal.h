// kvq_internal.h -- host-side launchers behind the C ABI of libkvq.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define KVQ_DEV_FLAG_SLOT_RANGE 1
#define KVQ_DEV_FLAG_KVLEN 2
#define KVQ_DEV_FLAG_POS_CAPACITY 4

namespace kvq {

enum { QM_INT8_TH = 0, QM_UINT4_TH = 1, QM_FP8E4M3_B32 = 2, QM_MXFP4_B32 = 3, QM_MXFP8_B32 = 4, QM_FP8E5M2_B32 = 5,
       QM_INT8_B32 = 6, QM_MXFP4E1M2_B32 = 7 };
enum { QF_MX_SCALE_OCP = 1 };   // quantize option (kvq.h KVQ_MX_SCALE_OCP)

hipError_t launch_quant_scatter(int qmode, bool bf16, const void* x, int B, int H, int T, int D,
                                int64_t sb, int64_t sh, int64_t st, const int32_t* slots,
                                int64_t ssb, int n_slots, uint8_t* codes, void* scales,
                                int8_t* zps, int flags, int32_t* err, hipStream_t s);

hipError_t launch_quant_scatter_kv(int qmode, bool bf16, const void* xk, const void* xv, int B, int H, int T, int D,
                                   int64_t sb, int64_t sh, int64_t st, const int32_t* slots, int64_t ssb,
                                   int n_slots, uint8_t* kcodes, void* kscales, int8_t* kzps, uint8_t* vcodes,
                                   void* vscales, int8_t* vzps, const int32_t* start_pos, int32_t* err,
                                   hipStream_t s);

hipError_t launch_positions_sink(const int32_t* start_pos, int T, int sink, int window, int32_t* slot_out,
                                 int32_t* cache_positions, int32_t* err, hipStream_t s);
hipError_t launch_positions_full(const int32_t* start_pos, int T, int capacity, int32_t* slot_out,
                                 int32_t* cache_positions, int32_t* err, hipStream_t s);
hipError_t launch_build_mask(const int32_t* cache_positions, int n_slots, const int32_t* start_pos, int Lq,
                             int sink, int window, float* mask, hipStream_t s);

struct DecodeLaunch {
    const void* q;
    bool q_bf16;
    int B, Hq, Hkv, S, D, qmode;
    const uint8_t* kc;
    const float* ks;
    const int8_t* kz;
    const uint8_t* vc;
    const float* vs;
    const int8_t* vz;
    const int32_t* kv_len;
    int kv_len_sb;          // 0: one kv_len for the batch; 1: kv_len[b]
    const float* mask;
    int64_t mask_sb;
    float sm_scale;
    void* out;
    bool out_bf16;
    int nsplit;
    float* part_o;
    float* part_ml;
    int32_t* err;
    unsigned* ctr = nullptr;   // single-pass kernel: per-plane tickets (zero between calls)
    // single-pass kernel, append variant (start_pos set): the new token's K
    // and V rows [B, Hkv, D] (element strides xsb, xsh) go to slot *start_pos
    // and kv_len is *start_pos + 1 (kv_len and mask unused)
    const int32_t* start_pos = nullptr;
    const void* xk = nullptr;
    const void* xv = nullptr;
    bool x_bf16 = false;
    int64_t xsb = 0, xsh = 0;
    // append variant, sink / ring layout (cpos set): the cache is sink +
    // window slots, cpos [n_slots] the slots' positions (in/out)
    int32_t* cpos = nullptr;
    int sink = 0, window = 0;
};

int decode_splits_max(int B, int Hq, int Hkv, int S, int D, int qmode);
int decode_splits(int B, int Hq, int Hkv, int S, int D, int qmode, bool qbf16);
hipError_t launch_sdpa_decode(const DecodeLaunch& L, hipStream_t s);

// Single-pass decode with the split merge in the same launch (int8
// per-token-head caches): which requests it runs, its split count, launch.
bool mfma_supported(int qmode, int D, int G, int S);
int mfma_splits_max(int B, int Hkv, int S, int D, int G);
int mfma_splits(int B, int Hkv, int S, int D, int G, bool qbf16);
hipError_t launch_sdpa_decode_mfma(const DecodeLaunch& L, hipStream_t s);

struct PrefillLaunch {
    const void* q;
    bool q_bf16;
    int B, Hq, Hkv, S, D, Lq, qmode;
    const uint8_t* kc;
    const float* ks;
    const int8_t* kz;
    const uint8_t* vc;
    const float* vs;
    const int8_t* vz;
    const int32_t* kv_len;
    int kv_len_sb;          // 0: one kv_len for the batch; 1: kv_len[b]
    const float* mask;
    bool causal;
    bool no_skip;
    float sm_scale;
    void* out;
    bool out_bf16;
    int32_t* err;
    int kv_splits = 1;      // > 1: key range split over workgroups, partials in part_o / part_ml
    float* part_o = nullptr;
    float* part_ml = nullptr;
};

hipError_t launch_sdpa_prefill(const PrefillLaunch& L, hipStream_t s);
int prefill_kv_splits(int B, int Hq, int Hkv, int Lq, int S);

// Merge per-split partials (o [rows, nsplit, D], (m, l) [rows, nsplit, 2],
// log2 units) into out [rows, D]; rows are (b, head) for decode and
// (b, head, query row) for a split prefill.
hipError_t launch_split_combine(int D, const float* part_o, const float* part_ml, int nsplit, int64_t rows,
                                void* out, bool out_bf16, hipStream_t s);

}  // namespace kvq
