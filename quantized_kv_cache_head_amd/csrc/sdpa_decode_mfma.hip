// sdpa_decode_mfma.hip -- single-pass decode attention (Lq = 1) over an int8
// per-token-head affine cache, both contractions on the int8 matrix cores,
// with the split merge in the same launch.
//
// What is computed: abaddon attention_cache, KvCache::forward_attention (q
// [batch, heads, q_len, head_dim], GQA expansion by repeat_kv, softmax scale)
// over the dequantized cache x = (code - zp) * scale (pytorch/executorch PR
// 24473, Summary: int8 entries, affine asymmetric per token and head, fp32
// scale, int8 zero point).  The key loop stops at the filled length kv_len, a
// device int32 scalar (PR 20351, kv_len note); ring and sink caches add a
// 0 / -inf float mask (PR 24473, Summary).  A slot the mask hides, or one at or
// past kv_len, takes no part: its codes and scales are never combined with
// anything, so unwritten slots may hold any bytes.
//
// Mapping on gfx950:
//  * Grid: B * Hkv planes (one (b, kv head)) times `ns` splits of NW waves.
//    Block ids are remapped so that the splits of a plane share an XCD (its
//    L2 then serves the plane's partials).  The plane's keys go in units of
//    64; unit u belongs to wave position (u mod NW ns) of the plane, the
//    positions running splits fastest, so the summation order depends on the
//    sizes only.
//  * Each wave keeps PD units in flight in its LDS ring (global_load_lds):
//    the K and V tiles [64 keys][D bytes] with 16-byte chunks placed by an
//    xor swizzle (so that the reads below meet no bank conflicts), then the
//    scales, mask values and zero points of the unit.  kv_len (a scalar
//    load) is waited for first: the copies then cover the wave's units only.
//  * q . k on v_mfma_i32_16x16x64_i8: A = q of the G heads as int8 limbs
//    (q * 2^e_h rounded to an integer of 22 bits, e_h per head, as three
//    balanced base-256 digits; two digits of 14 bits when G = 8), one MFMA row
//    per (head, digit); B = the raw signed K codes, 16 keys per MFMA.  Every
//    digit's sum is an exact int32; the zero point enters exactly per digit
//    as zp * sum(digits); the digits combine in fp32.
//  * Online softmax in the log2 domain on the MFMA output layout (lane =
//    key, lane group of 16 = head), with a running maximum per head that is
//    raised lazily (only when a score exceeds it by more than TAU: p <= 2^TAU).
//  * p * scale_v of the unit is quantized per head to 21-bit fixed point
//    relative to the unit's largest value (a power of two), three balanced
//    int8 digits again, and meets the V codes on the same int8 MFMA:
//    A = V^T (16 dims x 64 keys; the V tile is read as 32-bit words of 4 dims
//    and turned into 4 keys x 1 dim words by byte permutes), B = the digits of
//    (p * scale_v) [64 keys x (head, digit)].  The int32 results are scaled
//    into fp32 accumulators; the zero points enter as one correction per
//    head, sum p * scale_v * zp_v.
//  * Merge: the waves of a workgroup merge through LDS into one partial
//    (m, l, o) per head, written with device-coherent stores; the workgroup
//    then takes a ticket on the plane's counter, and the last one merges all
//    splits of the plane in split order, writes the output and sets the
//    counter back to zero.  With one split per plane (small caches) the
//    workgroup writes the output from its LDS merge: no partial, no ticket.
#include <type_traits>
#include <utility>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

template <typename T>
using mptr = const __attribute__((address_space(1))) T*;

template <typename T>
__device__ __forceinline__ mptr<T> wave_ptr(const T* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (mptr<T>)(((uint64_t)hi << 32) | lo);
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// DPP row_ror:n (rotate within each row of 16 lanes)
template <int N>
__device__ __forceinline__ float ror16(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, true));
}
// max / sum over the 16 lanes of each row; every lane gets the result
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, ror16<8>(v));
    v = fmaxf(v, ror16<4>(v));
    v = fmaxf(v, ror16<2>(v));
    return fmaxf(v, ror16<1>(v));
}
__device__ __forceinline__ float row_sum16(float v) {
    v += ror16<8>(v);
    v += ror16<4>(v);
    v += ror16<2>(v);
    return v + ror16<1>(v);
}

template <int... U, typename F>
__device__ __forceinline__ void for_each_unit(std::integer_sequence<int, U...>, F&& f) {
    (f(std::integral_constant<int, U>{}), ...);
}

// low byte as a signed digit
__device__ __forceinline__ int sext8(int x) { return (int)(int8_t)x; }

constexpr int MKEYS = 64;           // keys per unit
constexpr float MTAU = 8.0f;        // lazy rescale threshold (log2 units)

// Two waves per SIMD (eight per workgroup, four at D = 256), each with PD
// units in flight: while one wave waits for its copies (or for the copy
// engine to take more), the other computes.
template <int D>
struct MGeom {
    static constexpr int NW = D == 256 ? 4 : 8;           // waves per workgroup
    static constexpr int PD = 1;                          // units in flight per wave (ring slots)
    static constexpr int NT = 64 * NW;
    static constexpr int NH = D / 64;                     // 64-byte quarters of a row
    static constexpr int CPR = D / 16;                    // 16-byte chunks per row
    static constexpr int TILE = MKEYS * D;                // bytes of a K (or V) tile
    static constexpr int NKD = TILE / 1024;               // 16-byte copies per tile
    static constexpr int RPI = 1024 / D;                  // rows per copy
    static constexpr int OFF_V = TILE, OFF_M = 2 * TILE;  // V tile, metadata
    static constexpr int SLOT = 2 * TILE + 1024;
    static constexpr int NDMA = 2 * NKD + 4;              // copies per unit
    // chunk position of chunk c in row r: with these, 8 lanes reading the same
    // chunk of 8 consecutive rows (16-byte reads) and 32 lanes reading 16
    // consecutive words of rows r and r + 16 (4-byte reads) hit distinct banks
    __host__ __device__ static constexpr int sw(int r) { return D == 64 ? (r >> 1) & 3 : (r & 7) ^ (((r >> 4) & 1) << 2); }
};

template <int G>
struct MHeads {
    static constexpr int QL = G <= 4 ? 3 : 2;             // q digits
    static constexpr int RPH = QL == 3 ? 4 : 2;           // MFMA rows per head
    static constexpr int HPG = 4 / RPH;                   // heads per lane group (rows 4c .. 4c + 3)
    static constexpr int NPB = (3 * G + 15) / 16;         // 16-column blocks of (head, p digit)
    static constexpr float QMAXE = QL == 3 ? 22.0f : 14.0f;
};

}  // namespace

struct MfmaArgs {
    const void* q;
    int B, Hq, Hkv, S;
    const uint8_t* kc;
    const float* ks;
    const int8_t* kz;
    const uint8_t* vc;
    const float* vs;
    const int8_t* vz;
    const int32_t* kv_len;
    int kv_len_sb;
    const float* mask;
    int64_t mask_sb;
    float sm_scale_log2;   // sm_scale * log2(e)
    int ns;                // splits per plane
    unsigned* ctr;         // [B * Hkv] tickets, zero between calls
    float* part_ml;        // [B * Hkv, ns, G, 2]  (m, l)
    float* part_o;         // [B * Hkv, ns, G, D]
    void* out;
    int out_bf16;
    int32_t* err;
    // append variant: the new token's K and V rows x[b, kv head, :] (element
    // strides xsb, xsh), written at slot *start_pos of the full-context cache
    // and attended with kv_len = *start_pos + 1
    const void* xk;
    const void* xv;
    int x_bf16;
    int64_t xsb, xsh;
    const int32_t* start_pos;
    // sink / ring layout of the append variant (cpos set): the new slot is
    // p for p < sink, else sink + (p - sink) mod window (n_slots = sink +
    // window); cpos [n_slots] holds each slot's position (-1 empty) and
    // receives cpos[slot] = p; the mask word of a key is its position, made
    // visible (0) or not (-inf) by the additive-mask rule at query position
    // p; kv_len = min(p + 1, n_slots)
    int32_t* cpos;
    int sink, window;
};

// Affine int8 code parameters of one row spread over a wave (E elements per
// lane), with single IEEE fp32 operations in the order of the quant-scatter
// kernel, so scale, zero point and codes are bit-identical to it: lo = min(0,
// min x), hi = max(0, max x), scale = max((hi - lo) / 255, 2^-23), zp =
// clamp(-128 - rne(lo / scale)), code = clamp(rne(x / scale) + zp).
template <int E>
__device__ __forceinline__ void affine_row_codes(const float (&x)[E], int (&code)[E], float& scale, int& zp) {
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) { lo = fminf(lo, x[e]); hi = fmaxf(hi, x[e]); }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        lo = fminf(lo, __shfl_xor(lo, o, 64));
        hi = fmaxf(hi, __shfl_xor(hi, o, 64));
    }
    const float range = hi - lo;
    scale = fmaxf(range / 255.0f, 0x1p-23f);
    zp = min(max(-128 - (int)__builtin_rintf(lo / scale), -128), 127);
#pragma unroll
    for (int e = 0; e < E; ++e) code[e] = min(max((int)__builtin_rintf(x[e] / scale) + zp, -128), 127);
}

template <int D, int G, bool QBF16, bool APPEND>
__global__ __launch_bounds__(MGeom<D>::NT, 1) void sdpa_decode_mfma(MfmaArgs a) {
    using GM = MGeom<D>;
    using HM = MHeads<G>;
    constexpr int NW = GM::NW, NT = GM::NT, NH = GM::NH, CPR = GM::CPR, TILE = GM::TILE, NKD = GM::NKD;
    constexpr int RPI = GM::RPI, OFF_V = GM::OFF_V, OFF_M = GM::OFF_M, SLOT = GM::SLOT, NDMA = GM::NDMA;
    constexpr int QL = HM::QL, RPH = HM::RPH, HPG = HM::HPG, NPB = HM::NPB;
    constexpr int PD = GM::PD;
    constexpr float NEG_INF = -__builtin_huge_valf();
    constexpr float LOG2E = 1.4426950408889634f;
    static_assert(PD >= 1 && PD <= 3 && (PD - 1) * NDMA <= 63, "ring depth");
    static_assert(3 * G * D * 4 <= SLOT, "wave partial fits its ring slot");
    static_assert(!(D == 256 && G == 8), "D 256 with 8 heads per KV head runs the split kernel");

    // per wave: the q digits [16 rows][D] (read into registers before the key
    // loop), then, in the same bytes, the p digits of a unit [3 G rows]
    // [80 bytes] (the row pitch keeps 16-byte reads of 8 rows on distinct
    // banks).  No copy engine writes here.
    constexpr int PPITCH = 80;
    constexpr int PROWS = 3 * G > 16 ? 3 * G : 16;
    constexpr int QST = 16 * D > PROWS * PPITCH ? 16 * D : PROWS * PPITCH;
    // q of the group as copied in (every wave copies all of it and waits for
    // its own copies only: the bytes are the same)
    constexpr int QBYTES = G * D * (QBF16 ? 2 : 4);
    constexpr int NQD = (QBYTES + 1023) / 1024;
    __shared__ __attribute__((aligned(16))) uint8_t s_r0[NW * SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t s_r1[PD > 1 ? NW * SLOT : 16];
    __shared__ __attribute__((aligned(16))) uint8_t s_r2[PD > 2 ? NW * SLOT : 16];
    __shared__ __attribute__((aligned(16))) uint8_t s_q[NW][QST];
    __shared__ __attribute__((aligned(16))) uint8_t s_qin[NQD * 1024];
    __shared__ int s_qi[NW][G][4];                    // per head: digit sums, exponent
    __shared__ float s_m[NW][G], s_l[NW][G], s_c[NW][G];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the key loop is scalar
    const int n = lane & 15;                          // MFMA column: key of a tile / dim word
    const int c = lane >> 4;                          // lane group: MFMA rows 4c .. 4c + 3

    int bid = blockIdx.x;
    const int nwg = gridDim.x;
    if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
    const int ns = a.ns;
    const int plane = bid / ns;
    const int split = bid - plane * ns;
    const int b = plane / a.Hkv;
    const int g = plane - b * a.Hkv;
    const int S = a.S;

    const int64_t prow = (int64_t)plane * S;
    const mptr<uint8_t> kbase = wave_ptr(a.kc + prow * D);
    const mptr<uint8_t> vbase = wave_ptr(a.vc + prow * D);
    const mptr<float> ksb = wave_ptr(a.ks + prow);
    const mptr<float> vsb = wave_ptr(a.vs + prow);
    const mptr<uint32_t> kzw = (mptr<uint32_t>)wave_ptr(a.kz + prow);
    const mptr<uint32_t> vzw = (mptr<uint32_t>)wave_ptr(a.vz + prow);
    const bool has_mask = a.mask != nullptr;
    const mptr<float> mrow = has_mask ? wave_ptr(a.mask + (int64_t)b * a.mask_sb) : ksb;

    // waves of the plane, splits fastest: where a small cache has fewer units
    // than waves, the idle waves are spread over every workgroup of the plane
    const int W = ns * NW;
    const int wp = wave * ns + split;                 // this wave's position among them

    typedef const __attribute__((address_space(4))) int32_t* cptr_i32;
    int kv_len = S;
    int p_new = -1;                                   // slot this call writes (append variant)
    int qpos = 0;                                     // query position (sink / ring append)
    const bool sink_app = APPEND && a.cpos != nullptr;
    if constexpr (APPEND) {
        const int p = *(cptr_i32)(a.start_pos);
        qpos = p;
        if (sink_app) {
            // exactly the flags of the sink positions, the K+V scatter and a
            // decode with kv_len = min(p + 1, n_slots)
            if (p < 0) {
                if (a.err && split == 0 && tid == 0) atomicOr(a.err, KVQ_DEV_FLAG_SLOT_RANGE);
            } else {
                p_new = p < a.sink ? p : a.sink + (int)(((int64_t)p - a.sink) % a.window);
            }
            kv_len = p < S ? p + 1 : S;
        } else {
            // exactly the flags of the K+V full-context scatter followed by a
            // decode with kv_len = p + 1
            if (p < 0 || p >= S) {
                if (a.err && split == 0 && tid == 0) atomicOr(a.err, p < 0 ? KVQ_DEV_FLAG_SLOT_RANGE : KVQ_DEV_FLAG_POS_CAPACITY);
            } else {
                p_new = p;
            }
            kv_len = p < S ? p + 1 : S + 1;
        }
    } else {
        if (a.kv_len) kv_len = *(cptr_i32)(a.kv_len + (int64_t)b * a.kv_len_sb);
    }

    auto slot = [&](auto UC) __attribute__((always_inline)) -> uint8_t* {
        constexpr int U = decltype(UC)::value;
        if constexpr (U == 0) return s_r0 + wave * SLOT;
        else if constexpr (U == 1) return s_r1 + wave * SLOT;
        else return s_r2 + wave * SLOT;
    };
    typedef __attribute__((address_space(3))) void* lds_ptr;
    typedef const __attribute__((address_space(1))) void* glb_ptr;

    // per-lane parts of the copy addresses: tile copy j puts row RPI j + lane /
    // CPR, chunk (lane % CPR) ^ sw(row) at byte 1024 j + 16 lane of the tile
    const int crow = lane / CPR;
    const int cslot = lane % CPR;
    // metadata word i holds key 16 (i % 4) + i / 4, so that lane n finds the
    // keys n, 16 + n, 32 + n, 48 + n of the unit in words 4n .. 4n + 3
    const int mkey = 16 * (lane & 3) + (lane >> 2);
    // Asynchronous copies of unit t into ring slot U (live = false would read
    // row 0 instead).
    auto fetch = [&](auto UC, int t, bool live) __attribute__((always_inline)) {
        uint8_t* dst = slot(UC);
        const int row0 = (wp + t * W) * MKEYS;
        // the reads of the slot's previous unit have completed before the copies
        // that overwrite it are issued (a copy served from the L2 can land
        // before an LDS read still queued behind others)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NKD; ++j) {
            const int r = RPI * j + crow;
            const uint32_t grow = live ? (uint32_t)min(row0 + r, S - 1) : 0u;
            const uint32_t off = grow * D + 16u * (uint32_t)(cslot ^ GM::sw(r));
            __builtin_amdgcn_global_load_lds((glb_ptr)(kbase + off), (lds_ptr)(dst + 1024 * j), 16, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < NKD; ++j) {
            const int r = RPI * j + crow;
            const uint32_t grow = live ? (uint32_t)min(row0 + r, S - 1) : 0u;
            const uint32_t off = grow * D + 16u * (uint32_t)(cslot ^ GM::sw(r));
            __builtin_amdgcn_global_load_lds((glb_ptr)(vbase + off), (lds_ptr)(dst + OFF_V + 1024 * j), 16, 0, 0);
        }
        const uint32_t mr = live ? (uint32_t)min(row0 + mkey, S - 1) : 0u;
        __builtin_amdgcn_global_load_lds((glb_ptr)(ksb + mr), (lds_ptr)(dst + OFF_M), 4, 0, 0);
        __builtin_amdgcn_global_load_lds((glb_ptr)(vsb + mr), (lds_ptr)(dst + OFF_M + 256), 4, 0, 0);
        __builtin_amdgcn_global_load_lds((glb_ptr)(mrow + mr), (lds_ptr)(dst + OFF_M + 512), 4, 0, 0);
        // zero points: words [0, 16) K, [16, 32) V (lanes 32 .. 63 repeat V)
        const uint32_t zw = live ? (uint32_t)min(row0 / 4 + (lane & 15), S / 4 - 1) : 0u;
        const uint64_t za = lane < 16 ? (uint64_t)(kzw + zw) : (uint64_t)(vzw + zw);
        __builtin_amdgcn_global_load_lds((glb_ptr)za, (lds_ptr)(dst + OFF_M + 768), 4, 0, 0);
    };
    {
        const mptr<uint8_t> qg = wave_ptr(reinterpret_cast<const uint8_t*>(a.q) +
                                          ((int64_t)b * a.Hq + (int64_t)g * G) * D * (QBF16 ? 2 : 4));
#pragma unroll
        for (int j = 0; j < NQD; ++j)
            __builtin_amdgcn_global_load_lds((glb_ptr)(qg + min((j * 64 + lane) * 16, QBYTES - 16)),
                                             (lds_ptr)(&s_qin[1024 * j]), 16, 0, 0);
    }
    // append variant: every wave loads the plane's new K and V rows with q
    // (one round trip; which wave owns the new slot is known only later)
    // (raw words: every load is issued before any value is used)
    constexpr int XE = D / 64;                        // row elements per lane
    uint32_t xraw[2][XE];
    if constexpr (APPEND) {
        const int64_t xo = (int64_t)b * a.xsb + (int64_t)g * a.xsh + lane * XE;
        if (a.x_bf16) {
#pragma unroll
            for (int kv = 0; kv < 2; ++kv)
#pragma unroll
                for (int e = 0; e < XE; ++e)
                    xraw[kv][e] = reinterpret_cast<const uint16_t*>(kv ? a.xv : a.xk)[xo + e];
        } else {
#pragma unroll
            for (int kv = 0; kv < 2; ++kv)
#pragma unroll
                for (int e = 0; e < XE; ++e)
                    xraw[kv][e] = reinterpret_cast<const uint32_t*>(kv ? a.xv : a.xk)[xo + e];
        }
    }
    auto for_slots = [&](auto&& f) __attribute__((always_inline)) {
        for_each_unit(std::make_integer_sequence<int, PD>{}, f);
    };
    // Wait until at most the copies of `later` units (issued after the ones
    // waited for) are outstanding.  The wait is explicit: the compiler does
    // not track these copies.  Copies complete in issue order.
    auto wait_units = [&](int later) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        constexpr int N1 = NDMA, N2 = 2 * NDMA < 63 ? 2 * NDMA : 63, N3 = 3 * NDMA < 63 ? 3 * NDMA : 63;
        if (later >= 3) __builtin_amdgcn_s_waitcnt((N3 & 15) | ((N3 >> 4) << 14) | (7 << 4) | (15 << 8));
        else if (later == 2) __builtin_amdgcn_s_waitcnt((N2 & 15) | ((N2 >> 4) << 14) | (7 << 4) | (15 << 8));
        else if (later == 1) __builtin_amdgcn_s_waitcnt((N1 & 15) | ((N1 >> 4) << 14) | (7 << 4) | (15 << 8));
        else __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
        __builtin_amdgcn_sched_barrier(0);
    };
    // kv_len is known before any cache copy goes out: issued after the copies
    // of every wave of the chip, its load would return only once those had
    // been served, and no wave could start before.  The copies then cover
    // exactly the wave's units.
    if (kv_len < 1 || kv_len > S) {
        if (a.err && split == 0 && tid == 0) atomicOr(a.err, KVQ_DEV_FLAG_KVLEN);
        kv_len = kv_len < 1 ? 1 : S;
    }
    const int nunits = (kv_len + MKEYS - 1) / MKEYS;
    const int nsteps = wp < nunits ? (nunits - wp + W - 1) / W : 0;
    // Append variant: the new slot p_new (< kv_len) lies in unit u_new, which
    // belongs to wave u_new mod W at its step t_new.  That wave quantizes the
    // new K and V rows once its first copies are out, writes them to the
    // cache, and patches them (and, sink / ring, the slot's position) into
    // its tile once the unit's copies have landed, before any read of it.
    // No other wave reads the slot (clamped rows past the plane may read it
    // while it is written; they lie at or past kv_len and take no part).
    const int u_new = p_new >= 0 ? p_new / MKEYS : 0;
    const bool owner = APPEND && p_new >= 0 && u_new % W == wp;
    const int t_new = u_new / W;
    const int r_new = p_new - u_new * MKEYS;
    // the q copies were issued with the kv_len load and take about as long:
    // they have landed before the cache copies go out
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
    for_slots([&](auto UC) __attribute__((always_inline)) {
        constexpr int u = decltype(UC)::value;
        if (u < nsteps) fetch(UC, u, true);
    });
    int ncode[2][XE], nzp[2];
    float nscale[2];
    if constexpr (APPEND) {
        if (owner) {
            const int64_t crow = prow + p_new;
#pragma unroll
            for (int kv = 0; kv < 2; ++kv) {
                float xnew[XE];
#pragma unroll
                for (int e = 0; e < XE; ++e) xnew[e] = a.x_bf16 ? bf16_lo(xraw[kv][e]) : __uint_as_float(xraw[kv][e]);
                affine_row_codes<XE>(xnew, ncode[kv], nscale[kv], nzp[kv]);
                uint8_t* cg = const_cast<uint8_t*>(kv ? a.vc : a.kc) + crow * D + lane * XE;
#pragma unroll
                for (int e = 0; e < XE; ++e) cg[e] = (uint8_t)ncode[kv][e];
                if (lane == 0) {
                    const_cast<float*>(kv ? a.vs : a.ks)[crow] = nscale[kv];
                    const_cast<int8_t*>(kv ? a.vz : a.kz)[crow] = (int8_t)nzp[kv];
                }
            }
            // the slot's position (one writer: the owner of plane 0)
            if (sink_app && plane == 0 && lane == 0) a.cpos[p_new] = qpos;
        }
    }

    // ---- q digits ------------------------------------------------------------
    // Each wave converts the group on its own, through its own LDS words (no
    // workgroup barrier, which would wait for the cache copies in flight).
    // q as int8 digits: x = rne(q * 2^e_h), |x| < 2^22 (2^14 for two digits),
    // x = d0 + 256 d1 (+ 65536 d2) with every digit in [-128, 127].
    // lane l takes QPL consecutive elements of head l / LPH
    constexpr int LPH = 64 / G;
    constexpr int QPL = G * D / 64;
    const int hq = lane / LPH;
    const int e0 = (lane % LPH) * QPL;
    float csc[HPG];                                   // per own head: sm_scale log2(e) 2^-e_h
    int qs[HPG][QL];                                  // per own head and digit: sum over d
    i32x4_t qA[NH];                                   // MFMA A operand: digits of row n, d chunk 4 dq + c
    {
        float qv[QPL];
#pragma unroll
        for (int i = 0; i < QPL; ++i) {
            const int e = hq * D + e0 + i;
            if constexpr (QBF16) qv[i] = bf16_lo(reinterpret_cast<const uint16_t*>(s_qin)[e]);
            else qv[i] = reinterpret_cast<const float*>(s_qin)[e];
        }
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < QPL; ++i) mx = fmaxf(mx, fabsf(qv[i]));
#pragma unroll
        for (int o = 1; o < LPH; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        int qe = 0;
        if (mx > 0.0f) {
            int e;
            frexpf(mx, &e);                            // mx in [2^(e-1), 2^e)
            qe = (int)HM::QMAXE - e;                   // |q| 2^qe < 2^22 (2^14)
        }
        // zero rows first (rows of absent heads and the unused fourth digit)
        {
            constexpr int ZW = 16 * D / 16 / 64;       // 16-byte zero writes per lane
#pragma unroll
            for (int i = 0; i < ZW; ++i)
                reinterpret_cast<uint4*>(s_q[wave])[lane + 64 * i] = make_uint4(0u, 0u, 0u, 0u);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        int dsum[QL];
#pragma unroll
        for (int li = 0; li < QL; ++li) dsum[li] = 0;
        uint8_t dig[QL][QPL];
#pragma unroll
        for (int i = 0; i < QPL; ++i) {
            int x = (int)__builtin_rintf(ldexpf(qv[i], qe));
#pragma unroll
            for (int li = 0; li < QL; ++li) {
                const int dg = li == QL - 1 ? x : sext8(x);
                dsum[li] += dg;
                dig[li][i] = (uint8_t)dg;
                x = (x - dg) >> 8;
            }
        }
#pragma unroll
        for (int li = 0; li < QL; ++li) {
            uint32_t roff = (uint32_t)((hq * RPH + li) * D + e0);
            __asm__ volatile("" : "+v"(roff));             // see the tile reads in the key loop
            uint8_t* row = s_q[wave] + roff;
            if constexpr (QPL % 4 == 0) {
                // one store per 16 bytes (wider than the compiler would pair)
                uint32_t wd[QPL / 4];
#pragma unroll
                for (int w = 0; w < QPL / 4; ++w)
                    wd[w] = (uint32_t)dig[li][4 * w] | ((uint32_t)dig[li][4 * w + 1] << 8) |
                            ((uint32_t)dig[li][4 * w + 2] << 16) | ((uint32_t)dig[li][4 * w + 3] << 24);
                if constexpr (QPL == 4) {
                    *reinterpret_cast<uint32_t*>(row) = wd[0];
                } else if constexpr (QPL == 8) {
                    *reinterpret_cast<uint2*>(row) = make_uint2(wd[0], wd[1]);
                } else {
#pragma unroll
                    for (int w = 0; w < QPL / 4; w += 4)
                        *reinterpret_cast<uint4*>(row + 4 * w) = make_uint4(wd[w], wd[w + 1], wd[w + 2], wd[w + 3]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < QPL; ++i) row[i] = dig[li][i];
            }
#pragma unroll
            for (int o = 1; o < LPH; o <<= 1) dsum[li] += __shfl_xor(dsum[li], o, 64);
        }
        if (lane % LPH == 0) {
#pragma unroll
            for (int li = 0; li < QL; ++li) s_qi[wave][hq][li] = dsum[li];
            s_qi[wave][hq][3] = qe;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int dq = 0; dq < NH; ++dq) qA[dq] = *reinterpret_cast<const i32x4_t*>(s_q[wave] + n * D + 16 * (4 * dq + c));
#pragma unroll
        for (int j = 0; j < HPG; ++j) {
            const int h = min(c * HPG + j, G - 1);
#pragma unroll
            for (int li = 0; li < QL; ++li) qs[j][li] = s_qi[wave][h][li];
            csc[j] = ldexpf(a.sm_scale_log2, -s_qi[wave][h][3]);
        }
    }

    // ---- state ----------------------------------------------------------------
    // softmax per own head (lane group c owns heads c HPG + j); partial sums
    // of l and the zero-point correction are per lane until the end
    float m[HPG], l[HPG], corr[HPG];
#pragma unroll
    for (int j = 0; j < HPG; ++j) { m[j] = NEG_INF; l[j] = 0.0f; corr[j] = 0.0f; }
    // acc[pb][hh][e][i]: column 16 pb + n = (head, p digit), dim 64 hh + 16 c + 4 i + e
    float acc[NPB][NH][4][4];
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[pb][hh][e][i] = 0.0f;
    bool head_live[HPG];
#pragma unroll
    for (int j = 0; j < HPG; ++j) head_live[j] = c * HPG + j < G;
    // the (head, p digit) columns of this lane: head and digit
    int col_head[NPB], col_dig[NPB];
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
        const int col = 16 * pb + n;
        col_head[pb] = min(col / 3, G - 1);
        col_dig[pb] = col % 3;
    }
    uint8_t* const pbuf = s_q[wave];                 // the q digits are in registers now

    // value of lane group (h / HPG)'s slot h % HPG, for head h
    auto from_head = [&](const float* v, int h) __attribute__((always_inline)) -> float {
        const int src = 16 * (h / HPG);
        float r = __shfl(v[0], src, 64);
        if constexpr (HPG == 2) {
            const float r1 = __shfl(v[1], src, 64);
            r = (h & 1) ? r1 : r;
        }
        return r;
    };

    // unit t's copies have landed once at most the units t + 1 .. t + PD - 1
    // that exist are outstanding
    auto step = [&](auto UC, int t) __attribute__((always_inline)) {
        const int later = min(PD - 1, nsteps - 1 - t);
        wait_units(later);
        const uint8_t* src = slot(UC);
        if constexpr (APPEND) {
            if (owner && t == t_new) {
                // put the new rows in the tile where the copies put row r_new:
                // chunk c of the row at r_new D + 16 (c ^ sw(r_new)), the scales
                // in metadata word 4 (r_new % 16) + r_new / 16, the zero points
                // at byte r_new
                uint8_t* dst = const_cast<uint8_t*>(src);
#pragma unroll
                for (int kv = 0; kv < 2; ++kv) {
                    uint8_t* tl = dst + (kv ? OFF_V : 0) + r_new * D;
#pragma unroll
                    for (int e = 0; e < XE; ++e) {
                        const int d = lane * XE + e;
                        tl[16 * ((d >> 4) ^ GM::sw(r_new)) + (d & 15)] = (uint8_t)ncode[kv][e];
                    }
                    if (lane == 0) {
                        *reinterpret_cast<float*>(dst + OFF_M + 256 * kv + 4 * (4 * (r_new % 16) + r_new / 16)) =
                            nscale[kv];
                        dst[OFF_M + 768 + 64 * kv + r_new] = (uint8_t)(int8_t)nzp[kv];
                    }
                }
                if (sink_app && lane == 0)
                    *reinterpret_cast<int*>(dst + OFF_M + 512 + 4 * (4 * (r_new % 16) + r_new / 16)) = qpos;
                // the patch is read back by other lanes of the wave
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
        }
        const int row0 = (wp + t * W) * MKEYS;
        // ---- the unit's metadata; the K tile is read by the score MFMAs and
        // the V tile once the p digits are made, then the slot's refill goes
        // out, so that the next units stream in during the p.v half of the
        // work.  Each tile offset passes through an empty asm statement, so that the
        // compiler neither pairs nor hoists these reads: in the forms it makes
        // of them it loses which ring slot they read, and then waits for every
        // copy in flight, the other slots' included.
        const float4 sk4 = *reinterpret_cast<const float4*>(src + OFF_M + 16 * n);
        const float4 sv4 = *reinterpret_cast<const float4*>(src + OFF_M + 256 + 16 * n);
        const float4 mk4 = *reinterpret_cast<const float4*>(src + OFF_M + 512 + 16 * n);
        int zk[4], zv[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            zk[tt] = (int)reinterpret_cast<const int8_t*>(src + OFF_M + 768)[16 * tt + n];
            zv[tt] = (int)reinterpret_cast<const int8_t*>(src + OFF_M + 832)[16 * tt + n];
        }
        const float skv[4] = {sk4.x, sk4.y, sk4.z, sk4.w};
        const float svv[4] = {sv4.x, sv4.y, sv4.z, sv4.w};
        float mkv[4] = {mk4.x, mk4.y, mk4.z, mk4.w};
        if constexpr (APPEND) {
            if (sink_app) {
                // the mask words are the slots' positions: visible when
                // cp >= 0, cp <= p and (cp < sink or p - cp < window)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int cp = __float_as_int(mkv[tt]);
                    const bool vis = cp >= 0 && cp <= qpos && (cp < a.sink || qpos - cp < a.window);
                    mkv[tt] = vis ? 0.0f : NEG_INF;
                }
            }
        }
        // ---- scores: S^T[(head, digit)][key] for 4 tiles of 16 keys; the B
        // operand is K row 16 tt + n, 16-byte chunk 4 dq + c
        i32x4_t sc[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            sc[tt] = i32x4_t{0, 0, 0, 0};
#pragma unroll
            for (int dq = 0; dq < NH; ++dq) {
                const int kr = 16 * tt + n, cc = 4 * dq + c;
                uint32_t koff = (uint32_t)(kr * D + 16 * (cc ^ GM::sw(kr)));
                __asm__ volatile("" : "+v"(koff));
                const i32x4_t kb = *reinterpret_cast<const i32x4_t*>(src + koff);
                sc[tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qA[dq], kb, sc[tt], 0, 0, 0);
            }
        }
        float s[HPG][4];
        bool up = false;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int key = row0 + 16 * tt + n;
            const bool kv_ok = key < kv_len && !(has_mask && mkv[tt] == NEG_INF);
#pragma unroll
            for (int j = 0; j < HPG; ++j) {
                float sf;
                if constexpr (QL == 3) {
                    const int e0i = sc[tt][RPH * j] - zk[tt] * qs[j][0];
                    const int e1i = sc[tt][RPH * j + 1] - zk[tt] * qs[j][1];
                    const int e2i = sc[tt][RPH * j + 2] - zk[tt] * qs[j][2];
                    sf = fmaf((float)e2i, 65536.0f, fmaf((float)e1i, 256.0f, (float)e0i));
                } else {
                    const int e0i = sc[tt][RPH * j] - zk[tt] * qs[j][0];
                    const int e1i = sc[tt][RPH * j + 1] - zk[tt] * qs[j][1];
                    sf = fmaf((float)e1i, 256.0f, (float)e0i);
                }
                const bool ok = kv_ok && head_live[j];
                s[j][tt] = ok ? fmaf(sf, skv[tt] * csc[j], has_mask ? mkv[tt] * LOG2E : 0.0f) : NEG_INF;
                up |= s[j][tt] > m[j] + MTAU;
            }
        }
        if (__builtin_amdgcn_ballot_w64(up)) {
            // raise the running maxima (rare after the first unit)
            float alpha[HPG];
#pragma unroll
            for (int j = 0; j < HPG; ++j) {
                float mx = fmaxf(fmaxf(s[j][0], s[j][1]), fmaxf(s[j][2], s[j][3]));
                mx = row_max16(mx);
                const float mn = fmaxf(m[j], mx);
                alpha[j] = mn == NEG_INF ? 1.0f : __builtin_amdgcn_exp2f(m[j] - mn);
                m[j] = mn;
                l[j] *= alpha[j];
                corr[j] *= alpha[j];
            }
#pragma unroll
            for (int pb = 0; pb < NPB; ++pb) {
                const float ah = from_head(alpha, col_head[pb]);
#pragma unroll
                for (int hh = 0; hh < NH; ++hh)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[pb][hh][e][i] *= ah;
            }
        }
        // ---- p, p * scale_v and its digits
        float pv[HPG][4];
        float pmax[HPG];
#pragma unroll
        for (int j = 0; j < HPG; ++j) {
            pmax[j] = 0.0f;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const float p = s[j][tt] == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(s[j][tt] - m[j]);
                l[j] += p;
                pv[j][tt] = p == 0.0f ? 0.0f : p * svv[tt];
                corr[j] = fmaf(pv[j][tt], (float)zv[tt], corr[j]);
                pmax[j] = fmaxf(pmax[j], fabsf(pv[j][tt]));
            }
            pmax[j] = row_max16(pmax[j]);
        }
        // p * scale_v * 2^f < 2^21 per head, f from the unit's largest value
        float fsc[HPG];
#pragma unroll
        for (int j = 0; j < HPG; ++j) {
            int e = 0;
            if (pmax[j] > 0.0f) frexpf(pmax[j], &e);
            fsc[j] = (float)(21 - e);
        }
#pragma unroll
        for (int j = 0; j < HPG; ++j) {
            const int f = (int)fsc[j];
            uint32_t poff = (uint32_t)((3 * (c * HPG + j)) * PPITCH + n);
            __asm__ volatile("" : "+v"(poff));             // see the tile reads
            uint8_t* prow0 = pbuf + poff;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int x = (int)__builtin_rintf(ldexpf(pv[j][tt], f));
                const int x1 = (x - sext8(x)) >> 8;
                const int x2 = (x1 - sext8(x1)) >> 8;
                prow0[16 * tt] = (uint8_t)x;
                prow0[PPITCH + 16 * tt] = (uint8_t)x1;
                prow0[2 * PPITCH + 16 * tt] = (uint8_t)x2;
            }
        }
        // scale of this lane's columns: 256^digit 2^-f(head)
        float csv[NPB];
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) csv[pb] = ldexpf(1.0f, 8 * col_dig[pb] - (int)from_head(fsc, col_head[pb]));
        // the wave's own digit writes are read back below by other lanes of the
        // wave (one wave's LDS accesses are served in order)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        i32x4_t pB[NPB];
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb)   // (columns past 3 G read a row in use; their results are not used)
            pB[pb] = *reinterpret_cast<const i32x4_t*>(pbuf + min(16 * pb + n, PROWS - 1) * PPITCH + 16 * c);
        // V: words of 4 dims (dim word 16 hh + n) of the keys 16 c .. 16 c + 15
        auto read_v = [&](int hh, uint32_t* w) __attribute__((always_inline)) {
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                const int r = 16 * c + kk;
                const int dw = 16 * hh + n;
                uint32_t off = (uint32_t)(OFF_V + r * D + 16 * ((dw >> 2) ^ GM::sw(r)) + 4 * (dw & 3));
                __asm__ volatile("" : "+v"(off));
                w[kk] = *reinterpret_cast<const uint32_t*>(src + off);
            }
        };
        uint32_t vw[NH][16];
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) read_v(hh, vw[hh]);
        if (t + PD < nsteps) fetch(UC, t + PD, true);
        // ---- o^T[dim][(head, digit)] += V^T (p * scale_v digits)
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
            const uint32_t* w = vw[hh];
            // 4 x 4 byte transposes: op[e] word q4 = dim e of keys 4 q4 .. 4 q4 + 3
            i32x4_t op[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const uint32_t a0 = w[4 * q4], a1 = w[4 * q4 + 1], a2 = w[4 * q4 + 2], a3 = w[4 * q4 + 3];
                const uint32_t t0 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);
                const uint32_t t1 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);
                const uint32_t t2 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
                const uint32_t t3 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
                op[0][q4] = (int)__builtin_amdgcn_perm(t2, t0, 0x05040100u);
                op[1][q4] = (int)__builtin_amdgcn_perm(t2, t0, 0x07060302u);
                op[2][q4] = (int)__builtin_amdgcn_perm(t3, t1, 0x05040100u);
                op[3][q4] = (int)__builtin_amdgcn_perm(t3, t1, 0x07060302u);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int pb = 0; pb < NPB; ++pb) {
                    const i32x4_t r = __builtin_amdgcn_mfma_i32_16x16x64_i8(op[e], pB[pb], i32x4_t{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[pb][hh][e][i] = fmaf((float)r[i], csv[pb], acc[pb][hh][e][i]);
                }
        }
        // the digit buffer is rewritten by the next unit only after these reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // whole ring rounds (each step refills its slot with the unit PD later,
    // if the wave has it), then the rest of the ring
    int t0 = 0;
    for (; t0 + PD <= nsteps; t0 += PD) {
        for_slots([&](auto UC) __attribute__((always_inline)) {
            constexpr int u = decltype(UC)::value;
            step(UC, t0 + u);
        });
    }
    for_slots([&](auto UC) __attribute__((always_inline)) {
        constexpr int u = decltype(UC)::value;
        if (u < PD - 1 && t0 + u < nsteps) step(UC, t0 + u);
    });
    // every copy into the ring has landed before slot 0 is reused
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();

    // ---- the wave's partial -------------------------------------------------------
#pragma unroll
    for (int j = 0; j < HPG; ++j) {
        l[j] = row_sum16(l[j]);
        corr[j] = row_sum16(corr[j]);
    }
    // o columns (head, digit) x D, fp32, in the wave's slot-0 region
    float* s_ow = reinterpret_cast<float*>(s_r0 + wave * SLOT);
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
        const int col = 16 * pb + n;
        if (col < 3 * G) {
#pragma unroll
            for (int hh = 0; hh < NH; ++hh)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<float4*>(s_ow + col * D + 64 * hh + 16 * c + 4 * i) =
                        make_float4(acc[pb][hh][0][i], acc[pb][hh][1][i], acc[pb][hh][2][i], acc[pb][hh][3][i]);
        }
    }
    if (n == 0) {
#pragma unroll
        for (int j = 0; j < HPG; ++j) {
            const int h = c * HPG + j;
            if (h < G) {
                s_m[wave][h] = m[j];
                s_l[wave][h] = l[j];
                s_c[wave][h] = corr[j];
            }
        }
    }
    __syncthreads();

    // ---- one split per plane: the workgroup's merge is the result -------------
    constexpr int OPT = (G * D + NT - 1) / NT;
    if (ns == 1) {
#pragma unroll
        for (int i = 0; i < OPT; ++i) {
            const int idx = tid + NT * i;
            if (idx < G * D) {
                const int h = idx / D, d = idx % D;
                float M = NEG_INF;
#pragma unroll
                for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
                float o = 0.0f, lsum = 0.0f;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    const float fw = s_m[w][h] == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(s_m[w][h] - M);
                    const float* ow = reinterpret_cast<const float*>(s_r0 + w * SLOT);
                    const float ov = ow[(3 * h) * D + d] + ow[(3 * h + 1) * D + d] + ow[(3 * h + 2) * D + d] - s_c[w][h];
                    o = fmaf(fw, ov, o);
                    lsum = fmaf(fw, s_l[w][h], lsum);
                }
                // o + 0 as the split merge forms it (a -0 sum becomes +0), so
                // that the result does not depend on the split count's path
                const float res = lsum > 0.0f ? (o + 0.0f) / lsum : 0.0f;
                const int64_t oi = ((int64_t)b * a.Hq + (int64_t)g * G) * D + idx;
                if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_rne(res);
                else reinterpret_cast<float*>(a.out)[oi] = res;
            }
        }
        return;
    }

    // ---- the workgroup's partial: (m, l, o) per head ---------------------------
    float* pml = a.part_ml + ((int64_t)plane * ns + split) * G * 2;
    float* po = a.part_o + ((int64_t)plane * ns + split) * G * D;
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
        const int idx = tid + NT * i;
        if (idx < G * D) {
            const int h = idx / D, d = idx % D;
            float M = NEG_INF;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
            float o = 0.0f, lsum = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float fw = s_m[w][h] == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(s_m[w][h] - M);
                const float* ow = reinterpret_cast<const float*>(s_r0 + w * SLOT);
                const float ov = ow[(3 * h) * D + d] + ow[(3 * h + 1) * D + d] + ow[(3 * h + 2) * D + d] - s_c[w][h];
                o = fmaf(fw, ov, o);
                lsum = fmaf(fw, s_l[w][h], lsum);
            }
            __hip_atomic_store(po + idx, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (d == 0) {
                __hip_atomic_store(pml + 2 * h, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(pml + 2 * h + 1, lsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    // every partial store has completed (device-coherent) before the ticket
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const unsigned old = __hip_atomic_fetch_add(a.ctr + plane, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old == (unsigned)ns - 1;
        if (last) __hip_atomic_store(a.ctr + plane, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = last;
    }
    __syncthreads();
    if (!s_last) return;

    // ---- last workgroup of the plane: merge the splits in split order ---------
    const float* pml0 = a.part_ml + (int64_t)plane * ns * G * 2;
    const float* po0 = a.part_o + (int64_t)plane * ns * G * D;
    constexpr int CH = 8;
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
        const int idx = tid + NT * i;
        if (idx < G * D) {
            const int h = idx / D;
            float M = NEG_INF, lsum = 0.0f, o = 0.0f;
            for (int s0 = 0; s0 < ns; s0 += CH) {
                float mv[CH], lv[CH], ov[CH];
#pragma unroll
                for (int cI = 0; cI < CH; ++cI) {
                    const int sp = min(s0 + cI, ns - 1);
                    mv[cI] = __hip_atomic_load(pml0 + ((int64_t)sp * G + h) * 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    lv[cI] = __hip_atomic_load(pml0 + ((int64_t)sp * G + h) * 2 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    ov[cI] = __hip_atomic_load(po0 + (int64_t)sp * G * D + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                float mn = M;
#pragma unroll
                for (int cI = 0; cI < CH; ++cI)
                    if (s0 + cI < ns) mn = fmaxf(mn, mv[cI]);
                const float rsc = M == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(M - mn);
                o *= rsc;
                lsum *= rsc;
#pragma unroll
                for (int cI = 0; cI < CH; ++cI) {
                    const bool live = s0 + cI < ns && mv[cI] != NEG_INF;
                    const float wgt = live ? __builtin_amdgcn_exp2f(mv[cI] - mn) : 0.0f;
                    o = fmaf(wgt, ov[cI], o);
                    lsum = fmaf(wgt, lv[cI], lsum);
                }
                M = mn;
            }
            const float res = lsum > 0.0f ? o / lsum : 0.0f;
            const int64_t oi = ((int64_t)b * a.Hq + (int64_t)g * G) * D + idx;
            if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_rne(res);
            else reinterpret_cast<float*>(a.out)[oi] = res;
        }
    }
}


// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// Zero points are copied as aligned words of four keys, so the planes must
// keep them aligned (S % 4 == 0 and 4-byte aligned zero-point arrays; the
// caller checks the pointers).
// (D = 256 with 8 query heads per KV head would not fit the registers.)
bool mfma_supported(int qmode, int D, int G, int S) {
    return qmode == QM_INT8_TH && (D == 64 || D == 128 || D == 256) && (G == 1 || G == 2 || G == 4 || G == 8) &&
           !(D == 256 && G == 8) &&
           S % 4 == 0 && (int64_t)S * D < (int64_t(1) << 32);
}

static int mfma_nw(int D) { return D == 256 ? 4 : 8; }

// Splits per plane: one round of resident workgroups (one per CU), and no
// more than lets every wave of the plane get a unit of a full cache, except
// that a small cache may take up to eight splits as long as each workgroup
// keeps half its waves busy, a quarter for eight-wave workgroups once the
// plane has two units per wave of one workgroup (its units then spread over
// more CUs); at most 64.  `target` is the number of workgroups the device holds at once.
static int mfma_splits_for(int B, int Hkv, int S, int D, int target) {
    const int planes = B * Hkv;
    int ns = (target + planes - 1) / planes;
    const int units = S / MKEYS;
    int cap = units / mfma_nw(D);
    const int spread = (mfma_nw(D) == 8 && units >= 16) ? units / 2 : units / (mfma_nw(D) / 2);
    if (cap < 8) cap = spread < 8 ? spread : 8;
    if (cap > 64) cap = 64;
    if (cap < 1) cap = 1;
    if (ns > cap) ns = cap;
    return ns < 1 ? 1 : ns;
}

// Upper bound for sizing the workspace without a device: two workgroups on
// each of 256 CUs.
int mfma_splits_max(int B, int Hkv, int S, int D, int G) {
    (void)G;
    return mfma_splits_for(B, Hkv, S, D, 2 * 256);
}

int mfma_splits(int B, int Hkv, int S, int D, int G, bool qbf16) {
    (void)G;
    (void)qbf16;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0 || cus > 512)
        cus = 256;
    return mfma_splits_for(B, Hkv, S, D, cus);
}

template <int D, int G, bool QBF16>
static void launch_mfma_t(const MfmaArgs& a, int nwg, hipStream_t s) {
    if (a.start_pos) hipLaunchKernelGGL((sdpa_decode_mfma<D, G, QBF16, true>), dim3(nwg), dim3(MGeom<D>::NT), 0, s, a);
    else hipLaunchKernelGGL((sdpa_decode_mfma<D, G, QBF16, false>), dim3(nwg), dim3(MGeom<D>::NT), 0, s, a);
}

template <int D, bool QBF16>
static hipError_t launch_mfma_g(const MfmaArgs& a, int G, int nwg, hipStream_t s) {
    switch (G) {
    case 1: launch_mfma_t<D, 1, QBF16>(a, nwg, s); break;
    case 2: launch_mfma_t<D, 2, QBF16>(a, nwg, s); break;
    case 4: launch_mfma_t<D, 4, QBF16>(a, nwg, s); break;
    case 8:
        if constexpr (D == 256) return hipErrorInvalidValue;
        else launch_mfma_t<D, 8, QBF16>(a, nwg, s);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_sdpa_decode_mfma(const DecodeLaunch& L, hipStream_t s) {
    const int G = L.Hq / L.Hkv;
    MfmaArgs a{L.q, L.B, L.Hq, L.Hkv, L.S, L.kc, L.ks, L.kz, L.vc, L.vs, L.vz, L.kv_len, L.kv_len_sb, L.mask,
               L.mask_sb, L.sm_scale * 1.4426950408889634f, L.nsplit, L.ctr, L.part_ml, L.part_o, L.out,
               L.out_bf16 ? 1 : 0, L.err, L.xk, L.xv, L.x_bf16 ? 1 : 0, L.xsb, L.xsh, L.start_pos,
               L.cpos, L.sink, L.window};
    if (L.start_pos && (!L.xk || !L.xv)) return hipErrorInvalidValue;
    if (L.start_pos && (L.cpos ? (L.sink < 0 || L.window < 1 || L.sink + L.window != L.S) : L.mask != nullptr))
        return hipErrorInvalidValue;
    if (L.start_pos && L.cpos) {
        // the positions travel in the mask words (one row shared by the batch)
        a.mask = reinterpret_cast<const float*>(L.cpos);
        a.mask_sb = 0;
    }
    const int nwg = L.B * L.Hkv * L.nsplit;
    switch (L.D) {
    case 64: return L.q_bf16 ? launch_mfma_g<64, true>(a, G, nwg, s) : launch_mfma_g<64, false>(a, G, nwg, s);
    case 128: return L.q_bf16 ? launch_mfma_g<128, true>(a, G, nwg, s) : launch_mfma_g<128, false>(a, G, nwg, s);
    case 256: return L.q_bf16 ? launch_mfma_g<256, true>(a, G, nwg, s) : launch_mfma_g<256, false>(a, G, nwg, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
