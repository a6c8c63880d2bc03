// sdpa_decode_stream.hip -- single-pass decode attention (Lq = 1) over an
// int8 per-token-head affine cache, with the split merge in the same launch.
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
//  * Grid: B * Hkv planes (one (b, kv head)) times `ns` splits, one
//    workgroup of 4 waves each.  Consecutive block ids are spread over the 8
//    XCDs, so block ids are remapped to keep the splits of a plane on one XCD
//    (its L2 then serves the q and partial traffic of the plane).
//  * The plane's rows [0, kv_len) go in units of RS rows; unit u belongs to
//    wave (u mod 4 ns) of the plane, i.e. the units interleave over every
//    wave of every split.  The assignment depends on the sizes only, so the
//    summation order, and the result, is the same on every call.
//  * One pass: a wave step loads the K and V code rows of one unit, its
//    scales, zero points (and mask values) together, and keeps PD steps in
//    flight.  The first steps are issued before kv_len is known (rows are
//    clamped to the cache; rows past kv_len are dropped afterwards).
//  * A row's D code bytes are split over CL lanes of L bytes.  q . k uses
//    v_dot4_i32_i8 on the raw signed codes against q in two int8 limbs
//    (q * 2^k rounded to an integer of at most 14 bits plus sign, k chosen
//    per (b, kv head) from max |q|), so the dot product is an exact integer
//    sum; the zero point enters as zp * sum(q) in integers.  The lanes of a
//    row reduce-scatter their G partial dots, so that each lane ends with the
//    score of its own head(s).
//  * Online softmax in the log2 domain with a wave-uniform running maximum
//    per head that is raised lazily (only when a score exceeds it by more
//    than TAU, so p <= 2^TAU): the common step needs no cross-lane maximum.
//  * p * scale_v of each head is broadcast inside the row's lane group
//    (DPP or ds_swizzle) and every lane accumulates its L columns of V for
//    all G heads in fp32 FMAs on the sign-extended codes; the zero points
//    enter as one correction sum per head, sum p * scale_v * zp_v.
//  * Merge: the row slots of a wave are reduce-scattered with lane swaps,
//    then the waves of the workgroup merge through LDS into one partial
//    (m, l, o) per head.  The partial is written with device-coherent
//    stores; the workgroup then takes a ticket on the plane's counter, and
//    the last one to arrive merges all splits of the plane in split order
//    and writes the output (and sets the counter back to zero).
#include <type_traits>
#include <utility>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

template <typename T>
using gptr = const __attribute__((address_space(1))) T*;

template <typename T>
__device__ __forceinline__ gptr<T> uniform_ptr(const T* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (gptr<T>)(((uint64_t)hi << 32) | lo);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// DPP controls: quad_perm [1,0,3,2] (xor 1), quad_perm [2,3,0,1] (xor 2),
// row_half_mirror (lane i <-> 7 - i within 8), row_ror:4, row_ror:8 (xor 8
// within 16).
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_ROR4 = 0x124, DPP_ROR8 = 0x128;

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) { return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true); }
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Partner value across lane bit O inside a lane group (O = 1, 2, 4, 8): a
// pairing of the lanes with bit O clear and set that keeps the higher bits
// (xor for 1, 2, 8; the half mirror i <-> 7 - i for 4, which also changes the
// lower bits; every use below is a recursive halving, for which that is
// enough).
template <int O>
__device__ __forceinline__ int partner_i(int v) {
    if constexpr (O == 1) return dpp_i<DPP_XOR1>(v);
    else if constexpr (O == 2) return dpp_i<DPP_XOR2>(v);
    else if constexpr (O == 4) return dpp_i<DPP_HALF_MIRROR>(v);
    else return dpp_i<DPP_ROR8>(v);
}
template <int O>
__device__ __forceinline__ float partner_f(float v) { return __int_as_float(partner_i<O>(__float_as_int(v))); }

// Value of lane `src` of each aligned group of N lanes (N = 2, 4, 8, 16).
template <int N, int SRC>
__device__ __forceinline__ float group_bcast(float v) {
    if constexpr (N == 4) {
        return dpp_f<SRC | (SRC << 2) | (SRC << 4) | (SRC << 6)>(v);
    } else if constexpr (N == 2) {
        return dpp_f<SRC | (SRC << 2) | ((2 + SRC) << 4) | ((2 + SRC) << 6)>(v);
    } else {
        // ds_swizzle bit mode within 32 lanes: lane' = (lane & and) | or
        constexpr int AND = 0x1F & ~(N - 1);
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), AND | (SRC << 5)));
    }
}

// The same with the source position as a value that is a constant after
// unrolling (the switch folds away).
template <int N>
__device__ __forceinline__ float group_bcast_rt(float v, int src) {
    switch (src) {
    case 0: return group_bcast<N, 0>(v);
    case 1: return group_bcast<N, 1>(v);
    case 2: if constexpr (N > 2) return group_bcast<N, 2>(v); else return v;
    case 3: if constexpr (N > 2) return group_bcast<N, 3>(v); else return v;
    case 4: if constexpr (N > 4) return group_bcast<N, 4>(v); else return v;
    case 5: if constexpr (N > 4) return group_bcast<N, 5>(v); else return v;
    case 6: if constexpr (N > 4) return group_bcast<N, 6>(v); else return v;
    case 7: if constexpr (N > 4) return group_bcast<N, 7>(v); else return v;
    case 8: if constexpr (N > 8) return group_bcast<N, 8>(v); else return v;
    case 9: if constexpr (N > 8) return group_bcast<N, 9>(v); else return v;
    case 10: if constexpr (N > 8) return group_bcast<N, 10>(v); else return v;
    case 11: if constexpr (N > 8) return group_bcast<N, 11>(v); else return v;
    case 12: if constexpr (N > 8) return group_bcast<N, 12>(v); else return v;
    case 13: if constexpr (N > 8) return group_bcast<N, 13>(v); else return v;
    case 14: if constexpr (N > 8) return group_bcast<N, 14>(v); else return v;
    default: if constexpr (N > 8) return group_bcast<N, 15>(v); else return v;
    }
}

// Max / sum over the lanes of a wave that share their position in an aligned
// group of N lanes (lane bits >= log2 N); every lane gets the result.
template <int N, bool MAX>
__device__ __forceinline__ float across_groups(float v) {
    auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
    if constexpr (N <= 1) v = op(v, dpp_f<DPP_XOR1>(v));
    if constexpr (N <= 2) v = op(v, dpp_f<DPP_XOR2>(v));
    if constexpr (N <= 4) v = op(v, dpp_f<DPP_ROR4>(v));     // with the next: the 4 quads of a row
    if constexpr (N <= 8) v = op(v, dpp_f<DPP_ROR8>(v));
    {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// f(integral_constant<int, U>) for each U, in order, inlined.
template <int... U, typename F>
__device__ __forceinline__ void for_each_index(std::integer_sequence<int, U...>, F&& f) {
    (f(std::integral_constant<int, U>{}), ...);
}

// Lane geometry of one (D, G) instantiation.
#ifndef KVQ_SL4
#define KVQ_SL4 16
#endif
template <int D, int G, bool QBF16>
struct SGeom {
    // q in NQL balanced base-256 int8 limbs: two for bf16 q (16-bit fixed
    // point), three for fp32 q (24 bits)
    static constexpr int NQL = QBF16 ? 2 : 3;
    static constexpr int L = G <= 2 ? 32 : (G == 4 && QBF16) ? KVQ_SL4 : 16;   // code bytes of a row per lane
    static constexpr int CL = D / L;             // lanes per row
    static constexpr int RS = 64 / CL;           // rows per wave step
    static constexpr int NDW = L / 4;            // code dwords per lane
    static constexpr int NLD = L / 16;           // 16-byte loads per lane and row
    static constexpr int HPL = G >= CL ? G / CL : 1;   // heads whose softmax a lane runs
    static constexpr int NV = G * L;             // V accumulators per lane
    // lane position in its group -> first own head; head -> owner position
    __host__ __device__ static constexpr int own_head(int k, int j) { return G >= CL ? k * HPL + j : k / (CL / G); }
    __host__ __device__ static constexpr int owner_pos(int h) { return G >= CL ? h / HPL : h * (CL / G); }
    __host__ __device__ static constexpr int owner_slot(int h) { return G >= CL ? h % HPL : 0; }
};

#ifndef KVQ_SNW
#define KVQ_SNW 4
#endif
constexpr int SNW = KVQ_SNW;        // waves per workgroup
constexpr int SNT = 64 * SNW;       // threads per workgroup
#ifndef KVQ_SOCC
#define KVQ_SOCC 2
#endif
// workgroups per CU the kernel is built for (its registers allow that many
// waves per SIMD); the launch puts that many on each of the 256 CUs
__host__ __device__ constexpr int stream_occupancy(int G) { return G == 8 && KVQ_SOCC > 2 ? 2 : KVQ_SOCC; }
#ifndef KVQ_SPD
#define KVQ_SPD 4
#endif
constexpr int SPD = KVQ_SPD;        // wave steps in flight (LDS ring slots)
constexpr float STAU = 8.0f;        // lazy rescale threshold (log2 units)

// Reduce-scatter of the G integer dots of a row over its CL lanes (recursive
// halving from the top lane bit): afterwards lane position k holds the sums
// of its own heads SGeom::own_head(k, 0..HPL-1) in v[0..HPL).
template <int CL, int N, int O, typename T>
__device__ __forceinline__ void rs_dots(T* v, int k) {
    auto partner = [](T x) {
        if constexpr (sizeof(T) == 4 && T(0.5) != T(0)) return partner_f<O>(x);
        else return partner_i<O>(x);
    };
    if constexpr (O >= 1) {
        if constexpr (N > 1) {
            const bool up = (k & O) != 0;
#pragma unroll
            for (int i = 0; i < N / 2; ++i) {
                const T keep = up ? v[i + N / 2] : v[i];
                const T send = up ? v[i] : v[i + N / 2];
                v[i] = keep + partner(send);
            }
            rs_dots<CL, N / 2, O / 2, T>(v, k);
        } else {
            v[0] += partner(v[0]);
            rs_dots<CL, 1, O / 2, T>(v, k);
        }
    }
}

}  // namespace

struct StreamArgs {
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
};

template <int D, int G, bool QBF16>
__global__ __launch_bounds__(SNT, stream_occupancy(G)) void sdpa_decode_stream(StreamArgs a) {
    using GM = SGeom<D, G, QBF16>;
    constexpr int NQL = GM::NQL;
    constexpr int L = GM::L, CL = GM::CL, RS = GM::RS, NDW = GM::NDW, NLD = GM::NLD, HPL = GM::HPL, NV = GM::NV;
    constexpr int NW = SNW;

    constexpr float NEG_INF = -__builtin_huge_valf();
    constexpr float LOG2E = 1.4426950408889634f;
    static_assert(CL >= 2 && CL <= 16 && RS * CL == 64, "row split");
    // register reduce-scatter levels of the row slots (lane bits 5, 4 and, when
    // they are row bits, 3), then LDS
    constexpr int NLV = CL <= 8 ? 3 : 2;
    constexpr int NVR = NV >> NLV;
    constexpr int QE = G * D;                         // q elements of the group
    constexpr int QPL = QE / 64;                      // q elements per lane (every wave
                                                      // quantizes the whole group itself)
    static_assert(QE % 64 == 0, "q group");

    // LDS ring, one slot per step in flight, one region per wave: K codes
    // [NLD][64 lanes][16 B], V codes the same, then two 64-word metadata
    // blocks (scale_k, scale_v of the step's rows; mask values, zero-point
    // words).  Each slot is its own array, so a read of one slot waits only
    // for the copies into that slot.  Slot 0 later holds the wave's partial
    // accumulators.
    constexpr int OFF_V = NLD * 1024, OFF_M0 = 2 * NLD * 1024, OFF_M1 = OFF_M0 + 256;
    constexpr int SLOTB0 = OFF_M1 + 256;
    constexpr int NDMA = 2 * NLD + 2;                 // copies per step
    // wave steps in flight (LDS ring slots): SPD, or what the LDS of the
    // resident workgroups leaves room for (at least 2)
    constexpr int RING_BUDGET = (144 * 1024) / stream_occupancy(G);
    constexpr int PD_FIT = RING_BUDGET / (NW * SLOTB0);
    constexpr int PD = PD_FIT < 2 ? 2 : (PD_FIT < SPD ? PD_FIT : SPD);
    constexpr int SLOTB = SLOTB0 > NVR * 256 ? SLOTB0 : NVR * 256;   // bytes per wave, slot 0
    static_assert(PD >= 2 && PD <= 6, "ring depth");
    __shared__ __attribute__((aligned(16))) uint8_t s_r0[NW * SLOTB];
    __shared__ __attribute__((aligned(16))) uint8_t s_r1[NW * SLOTB0];
    __shared__ __attribute__((aligned(16))) uint8_t s_r2[PD > 2 ? NW * SLOTB0 : 16];
    __shared__ __attribute__((aligned(16))) uint8_t s_r3[PD > 3 ? NW * SLOTB0 : 16];
    __shared__ __attribute__((aligned(16))) uint8_t s_r4[PD > 4 ? NW * SLOTB0 : 16];
    __shared__ __attribute__((aligned(16))) uint8_t s_r5[PD > 5 ? NW * SLOTB0 : 16];
    // per wave: q as loaded (copied in by the wave itself), then overwritten by
    // its int8 limbs [limb][h][d]
    constexpr int QBYTES = QE * (QBF16 ? 2 : 4);
    constexpr int NQD = (QBYTES + 1023) / 1024;       // 16-byte copies per lane
    constexpr int QREG = NQD * 1024 > NQL * QE ? NQD * 1024 : NQL * QE;
    __shared__ __attribute__((aligned(16))) uint8_t s_q[NW][QREG];
    __shared__ float s_m[NW][G], s_l[NW][G], s_c[NW][G];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int k = lane % CL;                          // position in the row's lane group
    const int r = lane / CL;                          // row slot of the step

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
    const gptr<uint8_t> kbase = uniform_ptr(a.kc + prow * D);
    const gptr<uint8_t> vbase = uniform_ptr(a.vc + prow * D);
    const gptr<float> ksb = uniform_ptr(a.ks + prow);
    const gptr<float> vsb = uniform_ptr(a.vs + prow);
    const gptr<int8_t> kzb = uniform_ptr(a.kz + prow);
    const gptr<int8_t> vzb = uniform_ptr(a.vz + prow);
    const bool has_mask = a.mask != nullptr;
    const gptr<float> mrow = has_mask ? uniform_ptr(a.mask + (int64_t)b * a.mask_sb) : ksb;

    // units of this wave: wp, wp + W, wp + 2W, ...
    const int W = ns * NW;
    const int wp = split * NW + wave;

    // ---- kv_len (a scalar load: its wait does not wait for vector loads), the
    // q loads (whose wait then waits for nothing else), then the first PD steps
    // of the cache, before kv_len is known
    typedef const __attribute__((address_space(4))) int32_t* cptr_i32;
    int kv_len = a.kv_len ? *(cptr_i32)(a.kv_len + (int64_t)b * a.kv_len_sb) : S;
    // the wave's region of ring slot U (a compile-time index, so every access
    // names its own array)
    auto slot = [&](auto UC) __attribute__((always_inline)) -> uint8_t* {
        constexpr int U = decltype(UC)::value;
        if constexpr (U == 0) return s_r0 + wave * SLOTB;
        else if constexpr (U == 1) return s_r1 + wave * SLOTB0;
        else if constexpr (U == 2) return s_r2 + wave * SLOTB0;
        else if constexpr (U == 3) return s_r3 + wave * SLOTB0;
        else if constexpr (U == 4) return s_r4 + wave * SLOTB0;
        else return s_r5 + wave * SLOTB0;
    };
    typedef __attribute__((address_space(3))) void* lds_ptr;
    typedef const __attribute__((address_space(1))) void* glb_ptr;
    // zero points as aligned words of 4 rows (rows of a unit start on
    // multiples of RS >= 4; the host checks that the planes keep them aligned)
    const gptr<uint32_t> kzw = (gptr<uint32_t>)(gptr<uint8_t>)kzb;
    const gptr<uint32_t> vzw = (gptr<uint32_t>)(gptr<uint8_t>)vzb;
    const int lrow = lane % RS;                       // metadata lane -> row of the unit
    const int lsel = lane / RS;                       // metadata lane -> which array
    // Asynchronous copies of step t into ring slot u (global_load_lds: each
    // lane's bytes land at the slot region + lane * size).  A refill past the
    // wave's last step (live = false) reads one fixed line instead.
    auto fetch = [&](auto UC, int t, bool live) __attribute__((always_inline)) {
        uint8_t* dst = slot(UC);
        const int row0 = (wp + t * W) * RS;
        const uint32_t row = live ? (uint32_t)min(row0 + r, S - 1) : 0u;
        const uint32_t off = live ? row * D + (uint32_t)k * L : 0u;
#pragma unroll
        for (int c = 0; c < NLD; ++c)
            __builtin_amdgcn_global_load_lds((glb_ptr)(kbase + off + 16 * c), (lds_ptr)(dst + 1024 * c), 16, 0, 0);
#pragma unroll
        for (int c = 0; c < NLD; ++c)
            __builtin_amdgcn_global_load_lds((glb_ptr)(vbase + off + 16 * c), (lds_ptr)(dst + OFF_V + 1024 * c), 16, 0, 0);
        // metadata block 0: lanes [0, RS) scale_k, [RS, 2 RS) scale_v
        // (addresses picked with integer selects: no branch around the copies)
        const uint32_t mr = live ? (uint32_t)min(row0 + lrow, S - 1) : 0u;
        const uint64_t a_k = (uint64_t)(ksb + mr), a_v = (uint64_t)(vsb + mr), a_m = (uint64_t)(mrow + mr);
        const uint64_t m0 = lsel == 1 ? a_v : a_k;
        __builtin_amdgcn_global_load_lds((glb_ptr)m0, (lds_ptr)(dst + OFF_M0), 4, 0, 0);
        // block 1: [0, RS) mask values (the K scales when there is no mask),
        // then RS / 4 words of K zero points and RS / 4 of V zero points
        const int zi = lane - RS;                      // zero-point word index, K then V
        const uint32_t zw = live ? (uint32_t)min(row0 / 4 + (zi & (RS / 4 - 1)), S / 4 - 1) : 0u;
        const uint64_t a_zk = (uint64_t)(kzw + zw), a_zv = (uint64_t)(vzw + zw);
        const uint64_t m1 = lane < RS ? a_m : (zi < RS / 4 ? a_zk : a_zv);
        __builtin_amdgcn_global_load_lds((glb_ptr)m1, (lds_ptr)(dst + OFF_M1), 4, 0, 0);
    };
    {
        const gptr<uint8_t> qg = uniform_ptr(reinterpret_cast<const uint8_t*>(a.q) +
                                             ((int64_t)b * a.Hq + (int64_t)g * G) * D * (QBF16 ? 2 : 4));
#pragma unroll
        for (int j = 0; j < NQD; ++j)
            __builtin_amdgcn_global_load_lds((glb_ptr)(qg + min((j * 64 + lane) * 16, QBYTES - 16)),
                                             (lds_ptr)(&s_q[wave][1024 * j]), 16, 0, 0);
    }
    auto for_slots = [&](auto&& f) __attribute__((always_inline)) {   // f(integral_constant<int, u>), u < PD
        for_each_index(std::make_integer_sequence<int, PD>{}, f);
    };
    // The first step goes out before kv_len is known (a speculative copy of
    // rows that may lie past it); the others only where the wave has steps.
#ifndef KVQ_SPEC
#define KVQ_SPEC 4
#endif
    for_slots([&](auto UC) __attribute__((always_inline)) {
        if constexpr (decltype(UC)::value < KVQ_SPEC) fetch(UC, decltype(UC)::value, true);
    });
    if (kv_len < 1 || kv_len > S) {
        if (a.err && split == 0 && tid == 0) atomicOr(a.err, KVQ_DEV_FLAG_KVLEN);
        kv_len = kv_len < 1 ? 1 : S;
    }
    const int nunits = (kv_len + RS - 1) / RS;
    const int nsteps = wp < nunits ? (nunits - wp + W - 1) / W : 0;
    for_slots([&](auto UC) __attribute__((always_inline)) {
        constexpr int u = decltype(UC)::value;
        if constexpr (u >= KVQ_SPEC) fetch(UC, u, u < nsteps);
    });


    // ---- q: int8 limbs of q * 2^qk ------------------------------------------
    // Every wave quantizes the whole group on its own (the same values in each
    // wave) and passes the digits through its own LDS words: no workgroup
    // barrier, which would wait for the cache copies in flight.
    // q_int = rne(q * 2^qk) in balanced base-256 digits l_0 + 256 l_1 (+ 65536
    // l_2), each in [-128, 127]: |q_int| <= QIMAX, max |q| * 2^qk in
    // [QIMAX / 2, QIMAX]
    constexpr float QIMAX = NQL == 2 ? 32639.0f : 8355711.0f;
    int qk = 0;
    {
        // the q copies were issued before the PD steps of cache copies
        constexpr int LATER = PD * NDMA;
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt((LATER & 15) | ((LATER >> 4) << 14) | (7 << 4) | (15 << 8));
        __builtin_amdgcn_sched_barrier(0);
        float qv[QPL];
#pragma unroll
        for (int i = 0; i < QPL; ++i) {
            const int e = lane * QPL + i;
            if constexpr (QBF16) qv[i] = bf16_lo(reinterpret_cast<const uint16_t*>(s_q[wave])[e]);
            else qv[i] = reinterpret_cast<const float*>(s_q[wave])[e];
        }
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < QPL; ++i) mx = fmaxf(mx, fabsf(qv[i]));
        mx = across_groups<1, true>(mx);
        // every lane's q reads are served before the limbs overwrite them
        __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (mx > 0.0f) {
            int e;
            frexpf(mx, &e);                            // mx in [2^(e-1), 2^e)
            qk = (NQL == 2 ? 15 : 23) - e;
            if (ldexpf(mx, qk) > QIMAX) qk -= 1;
        }
#pragma unroll
        for (int i = 0; i < QPL; ++i) {
            const int e = lane * QPL + i;
            int qi = (int)__builtin_rintf(ldexpf(qv[i], qk));
#pragma unroll
            for (int li = 0; li < NQL; ++li) {
                const int dg = li == NQL - 1 ? qi : (int)(int8_t)qi;   // low digit in [-128, 127]
                reinterpret_cast<int8_t*>(s_q[wave])[li * QE + e] = (int8_t)dg;
                qi = (qi - dg) >> 8;
            }
        }
    }
    // the wave's own LDS writes are done before its reads (one wave's LDS
    // accesses are served in order; the fence keeps the compiler from moving them)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // limbs [NQL - NQR, NQL) stay in registers; the lower ones are read from
    // the wave's LDS words at every step
#ifndef KVQ_QREG
#define KVQ_QREG 3
#endif
    constexpr int NQR = KVQ_QREG < NQL ? KVQ_QREG : NQL;
    uint32_t qw[NQL][G][NDW];
#pragma unroll
    for (int li = 0; li < NQL; ++li)
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < NDW; ++i)
                qw[li][h][i] = reinterpret_cast<const uint32_t*>(s_q[wave])[(li * QE + h * D) / 4 + k * NDW + i];
    // per own head: sum_d q_int (exact integer for two limbs; for three, the
    // fp32 value of 65536 S2 + 256 S1 + S0), from the lane's own digits (byte
    // sums by v_dot4 against ones) summed over the row's lanes
    int qsum[HPL];
    float qsumf[HPL];
    {
        int qs[NQL][G];
#pragma unroll
        for (int li = 0; li < NQL; ++li)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                int x = 0;
#pragma unroll
                for (int i = 0; i < NDW; ++i) x = __builtin_amdgcn_sdot4((int)qw[li][h][i], 0x01010101, x, false);
                if constexpr (CL >= 2) x += dpp_i<DPP_XOR1>(x);
                if constexpr (CL >= 4) x += dpp_i<DPP_XOR2>(x);
                if constexpr (CL >= 8) x += dpp_i<DPP_HALF_MIRROR>(x);
                if constexpr (CL >= 16) x += dpp_i<DPP_ROR8>(x);
                qs[li][h] = x;
            }
#pragma unroll
        for (int j = 0; j < HPL; ++j) {
            int s0 = 0, s1 = 0, s2 = 0;
#pragma unroll
            for (int h = 0; h < G; ++h)
                if (h == GM::own_head(k, j)) {
                    s0 = qs[0][h];
                    s1 = qs[1][h];
                    s2 = qs[NQL - 1][h];
                }
            qsum[j] = s0 + 256 * s1;
            qsumf[j] = NQL == 3 ? fmaf((float)s2, 65536.0f, fmaf((float)s1, 256.0f, (float)s0)) : 0.0f;
        }
    }
    const float csc = ldexpf(a.sm_scale_log2, -qk);


    float m[HPL], l[HPL], corr[HPL];
#pragma unroll
    for (int j = 0; j < HPL; ++j) { m[j] = NEG_INF; l[j] = 0.0f; corr[j] = 0.0f; }
    float acc[G][L];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < L; ++e) acc[h][e] = 0.0f;

    // The copies of a step must have landed before its slot is read.  The
    // wait is explicit (the compiler does not track these copies): copies
    // complete in issue order, so allowing the `later` steps issued after
    // this one to be outstanding, `later` * NDMA copies, is enough; any other
    // memory operation in between only makes the wait stricter.
    auto wait_copies = [&](int later) __attribute__((always_inline)) {
        const int n = later * NDMA;                   // <= 5 * 6 < 64
        __builtin_amdgcn_sched_barrier(0);
        switch (n) {
#define KVQ_VMW(N) case N: __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8)); break;
        KVQ_VMW(0) KVQ_VMW(4) KVQ_VMW(6) KVQ_VMW(8) KVQ_VMW(12) KVQ_VMW(16) KVQ_VMW(18) KVQ_VMW(20) KVQ_VMW(24)
        KVQ_VMW(30)
#undef KVQ_VMW
        default: __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); break;   // vmcnt(0)
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    auto step = [&](auto UC, int t, int later) __attribute__((always_inline)) {
        wait_copies(later);
        const uint8_t* src = slot(UC);
        uint4 kb[NLD], vb[NLD];
#pragma unroll
        for (int c = 0; c < NLD; ++c) {
            kb[c] = *reinterpret_cast<const uint4*>(src + 1024 * c + 16 * lane);
            vb[c] = *reinterpret_cast<const uint4*>(src + OFF_V + 1024 * c + 16 * lane);
        }
        const float msk = reinterpret_cast<const float*>(src + OFF_M0)[r];
        const float msv = reinterpret_cast<const float*>(src + OFF_M0)[RS + r];
        const float mmk = reinterpret_cast<const float*>(src + OFF_M1)[r];
        const int mzk = (int)(int8_t)(reinterpret_cast<const uint32_t*>(src + OFF_M1)[RS + r / 4] >> (8 * (r % 4)));
        const int mzv = (int)(int8_t)(reinterpret_cast<const uint32_t*>(src + OFF_M1)[RS + RS / 4 + r / 4] >> (8 * (r % 4)));
        // q . codes per limb in exact integers (v_dot4_i32_i8 on the raw signed
        // codes), then per row: sum over the lanes of the row (reduce-scatter)
        // and the zero point as zp * sum(q_int)
        int dsum[NQL][G];
#pragma unroll
        for (int li = 0; li < NQL; ++li)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                int acc_i = 0;
#pragma unroll
                for (int c = 0; c < NLD; ++c) {
                    const uint32_t w4[4] = {kb[c].x, kb[c].y, kb[c].z, kb[c].w};
                    uint32_t q4[4];
                    if (li >= NQL - NQR) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) q4[i] = qw[li][h][4 * c + i];
                    } else {
                        const uint4 x = reinterpret_cast<const uint4*>(s_q[wave])[((li * QE + h * D) / 4 + k * NDW) / 4 + c];
                        q4[0] = x.x; q4[1] = x.y; q4[2] = x.z; q4[3] = x.w;
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc_i = __builtin_amdgcn_sdot4((int)q4[i], (int)w4[i], acc_i, false);
                }
                dsum[li][h] = acc_i;
            }
        float sdot[HPL];
        if constexpr (NQL == 2) {
            // |q_int| < 2^15, |code - zp| <= 255, D <= 256: every sum fits int32
            int dts[G];
#pragma unroll
            for (int h = 0; h < G; ++h) dts[h] = dsum[0][h] + 256 * dsum[1][h];
            rs_dots<CL, G, CL / 2, int>(dts, k);
#pragma unroll
            for (int j = 0; j < HPL; ++j)
                sdot[j] = (float)(int)((uint32_t)dts[j] - (uint32_t)(mzk * qsum[j]));
        } else {
            float dtf[G];
#pragma unroll
            for (int h = 0; h < G; ++h)
                dtf[h] = fmaf((float)dsum[2][h], 65536.0f, fmaf((float)dsum[1][h], 256.0f, (float)dsum[0][h]));
            rs_dots<CL, G, CL / 2, float>(dtf, k);
#pragma unroll
            for (int j = 0; j < HPL; ++j) sdot[j] = fmaf(-(float)mzk, qsumf[j], dtf[j]);
        }
        const int row = (wp + t * W) * RS + r;
        const bool valid = row < kv_len && !(has_mask && mmk == NEG_INF);
        const float sk = msk * csc;
        float s[HPL];
        bool up = false;
#pragma unroll
        for (int j = 0; j < HPL; ++j) {
            s[j] = valid ? fmaf(sdot[j], sk, has_mask ? mmk * LOG2E : 0.0f) : NEG_INF;
            up |= s[j] > m[j] + STAU;
        }
        if (__builtin_amdgcn_ballot_w64(up)) {
            // raise the running maxima of the wave (rare after the first step)
            float alpha[HPL];
#pragma unroll
            for (int j = 0; j < HPL; ++j) {
                const float mn = fmaxf(m[j], across_groups<CL, true>(s[j]));
                alpha[j] = mn == NEG_INF ? 1.0f : __builtin_amdgcn_exp2f(m[j] - mn);
                m[j] = mn;
                l[j] *= alpha[j];
                corr[j] *= alpha[j];
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float ah = group_bcast_rt<CL>(alpha[GM::owner_slot(h)], GM::owner_pos(h));
#pragma unroll
                for (int e = 0; e < L; ++e) acc[h][e] *= ah;
            }
        }
        float pv[HPL];
#pragma unroll
        for (int j = 0; j < HPL; ++j) {
            const float p = valid ? __builtin_amdgcn_exp2f(s[j] - m[j]) : 0.0f;
            l[j] += p;
            pv[j] = valid ? p * msv : 0.0f;
            corr[j] = fmaf(pv[j], (float)mzv, corr[j]);
        }
        float pb[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pb[h] = group_bcast_rt<CL>(pv[GM::owner_slot(h)], GM::owner_pos(h));
#pragma unroll
        for (int c = 0; c < NLD; ++c) {
            const uint32_t w4[4] = {vb[c].x, vb[c].y, vb[c].z, vb[c].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float f[4];
                f[0] = (float)(int8_t)(w4[i]);
                f[1] = (float)(int8_t)(w4[i] >> 8);
                f[2] = (float)(int8_t)(w4[i] >> 16);
                f[3] = (float)(int8_t)(w4[i] >> 24);
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[h][16 * c + 4 * i + e] = fmaf(pb[h], f[e], acc[h][16 * c + 4 * i + e]);
            }
        }
    };

    // whole ring rounds: every slot is refilled right after it is used (a
    // refill past the wave's last step reads one fixed line; no branch around
    // the copies keeps the wait counts exact), then the rest of the ring
    // without refills
    int t0 = 0;
    for (; t0 + PD <= nsteps; t0 += PD) {
        // issue priority falls as the wave gets through its steps, so that the
        // waves sharing a SIMD keep pace with each other (otherwise the
        // younger workgroup of a CU lags and finishes alone)
        switch ((4 * t0) / nsteps) {
        case 0: __builtin_amdgcn_s_setprio(3); break;
        case 1: __builtin_amdgcn_s_setprio(2); break;
        case 2: __builtin_amdgcn_s_setprio(1); break;
        default: __builtin_amdgcn_s_setprio(0); break;
        }
        for_slots([&](auto UC) __attribute__((always_inline)) {
            constexpr int u = decltype(UC)::value;
            step(UC, t0 + u, PD - 1);
            fetch(UC, t0 + u + PD, t0 + u + PD < nsteps);
        });
    }
    for_slots([&](auto UC) __attribute__((always_inline)) {
        constexpr int u = decltype(UC)::value;
        if (u < PD - 1 && t0 + u < nsteps) step(UC, t0 + u, PD - 1 - u);
    });
    __builtin_amdgcn_s_setprio(0);
    // every copy into the ring has landed before slot 0 is reused
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();

    // ---- merge the row slots of the wave --------------------------------------
    // l and the zero-point correction: sums over the lanes of each head
#pragma unroll
    for (int j = 0; j < HPL; ++j) {
        l[j] = across_groups<CL, false>(l[j]);
        corr[j] = across_groups<CL, false>(corr[j]);
    }
    float av[NV];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < L; ++e) av[h * L + e] = acc[h][e];
    // reduce-scatter over lane bits 5, 4 (and 3): the upper half of the
    // values stays where the bit is set
    {
        constexpr int N1 = NV / 2;
#pragma unroll
        for (int i = 0; i < N1; ++i) {
            // lanes 0..31 end with the lower halves of lanes l and l + 32,
            // lanes 32..63 with the upper halves
            auto rr = __builtin_amdgcn_permlane32_swap(__float_as_uint(av[i]), __float_as_uint(av[i + N1]), false, false);
            av[i] = __uint_as_float(rr[0]) + __uint_as_float(rr[1]);
        }
    }
    {
        constexpr int N2 = NV / 4;
#pragma unroll
        for (int i = 0; i < N2; ++i) {
            auto rr = __builtin_amdgcn_permlane16_swap(__float_as_uint(av[i]), __float_as_uint(av[i + N2]), false, false);
            av[i] = __uint_as_float(rr[0]) + __uint_as_float(rr[1]);
        }
    }
    if constexpr (NLV == 3) {
        constexpr int N3 = NV / 8;
        const bool up = (lane & 8) != 0;
#pragma unroll
        for (int i = 0; i < N3; ++i) {
            const float keep = up ? av[i + N3] : av[i];
            const float send = up ? av[i] : av[i + N3];
            av[i] = keep + dpp_f<DPP_ROR8>(send);
        }
    }
    float* s_accw = reinterpret_cast<float*>(s_r0 + wave * SLOTB);   // [64][NVR] of this wave
#pragma unroll
    for (int i = 0; i < NVR; ++i) s_accw[lane * NVR + i] = av[i];
    if (r == 0) {
#pragma unroll
        for (int j = 0; j < HPL; ++j) {
            const int h = GM::own_head(k, j);
            if (k == GM::owner_pos(h)) {
                s_m[wave][h] = m[j];
                s_l[wave][h] = l[j];
                s_c[wave][h] = corr[j];
            }
        }
    }
    __syncthreads();

    // ---- the workgroup's partial: (m, l, o) per head ---------------------------
    constexpr int OPT = (G * D + SNT - 1) / SNT;      // outputs per thread
    float* pml = a.part_ml + ((int64_t)plane * ns + split) * G * 2;
    float* po = a.part_o + ((int64_t)plane * ns + split) * G * D;
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
        const int idx = tid + SNT * i;
        if (idx < G * D) {
            const int h = idx / D, d = idx % D;
            float M = NEG_INF;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
            const int kk = d / L, e = d % L;
            const int v = h * L + e;
            const int blk = v / NVR, jj = v % NVR;      // value block -> lane bits 5,4(,3)
            float o = 0.0f, lsum = 0.0f, csum = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float fw = s_m[w][h] == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(s_m[w][h] - M);
                float ow = 0.0f;
                if constexpr (NLV == 3) {
                    // lanes: bits 5,4,3 = blk; bits [log2 CL, 3) free row bits; low bits = kk
                    constexpr int FREE = 8 / CL;
#pragma unroll
                    for (int fr = 0; fr < FREE; ++fr) ow += reinterpret_cast<const float*>(s_r0 + w * SLOTB)[(blk * 8 + fr * CL + kk) * NVR + jj];
                } else {
                    ow = reinterpret_cast<const float*>(s_r0 + w * SLOTB)[(blk * 16 + kk) * NVR + jj];
                }
                o = fmaf(fw, ow, o);
                lsum = fmaf(fw, s_l[w][h], lsum);
                csum = fmaf(fw, s_c[w][h], csum);
            }
            o -= csum;
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
        const int idx = tid + SNT * i;
        if (idx < G * D) {
            const int h = idx / D;
            float M = NEG_INF, lsum = 0.0f, o = 0.0f;
            for (int s0 = 0; s0 < ns; s0 += CH) {
                float mv[CH], lv[CH], ov[CH];
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    const int sp = min(s0 + c, ns - 1);
                    mv[c] = __hip_atomic_load(pml0 + ((int64_t)sp * G + h) * 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    lv[c] = __hip_atomic_load(pml0 + ((int64_t)sp * G + h) * 2 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    ov[c] = __hip_atomic_load(po0 + (int64_t)sp * G * D + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                float mn = M;
#pragma unroll
                for (int c = 0; c < CH; ++c)
                    if (s0 + c < ns) mn = fmaxf(mn, mv[c]);
                const float rsc = M == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(M - mn);
                o *= rsc;
                lsum *= rsc;
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    const bool live = s0 + c < ns && mv[c] != NEG_INF;
                    const float wgt = live ? __builtin_amdgcn_exp2f(mv[c] - mn) : 0.0f;
                    o = fmaf(wgt, ov[c], o);
                    lsum = fmaf(wgt, lv[c], lsum);
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

static int stream_rs(int D, int G) { return 64 / (D / (G <= 4 ? 32 : 16)); }

// Zero points are copied as aligned words of four rows, so the planes must
// keep them aligned (S % 4 == 0 and 4-byte aligned zero-point arrays; the
// caller checks the pointers).
bool stream_supported(int qmode, int D, int G, int S) {
    return qmode == QM_INT8_TH && (D == 64 || D == 128 || D == 256) && (G == 1 || G == 2 || G == 4 || G == 8) &&
           S % 4 == 0 && (int64_t)S * D < (int64_t(1) << 32);
}

// Splits per plane: one round of resident workgroups, and no more than every
// wave of the plane can get a unit of a full cache; at most 64.  The upper
// bound (3 workgroups on each of 256 CUs) sizes the workspace without a
// device; a launch uses what its instantiation's registers and LDS let the
// device hold at once.
static int splits_for(int B, int Hkv, int S, int D, int G, int target) {
    const int planes = B * Hkv;
    int ns = (target + planes - 1) / planes;
    int cap = S / (SNW * stream_rs(D, G));
    if (cap > 64) cap = 64;
    if (cap < 1) cap = 1;
    if (ns > cap) ns = cap;
    return ns < 1 ? 1 : ns;
}

int stream_splits_max(int B, int Hkv, int S, int D, int G) { return splits_for(B, Hkv, S, D, G, 3 * 256 * 4 / SNW); }

template <int D, int G, bool QBF16>
static const void* stream_kernel() { return reinterpret_cast<const void*>(&sdpa_decode_stream<D, G, QBF16>); }

static const void* stream_kernel_for(int D, int G, bool qbf16) {
#define KVQ_SKG(DD)                                                                                  \
    switch (G) {                                                                                     \
    case 1: return qbf16 ? stream_kernel<DD, 1, true>() : stream_kernel<DD, 1, false>();             \
    case 2: return qbf16 ? stream_kernel<DD, 2, true>() : stream_kernel<DD, 2, false>();             \
    case 4: return qbf16 ? stream_kernel<DD, 4, true>() : stream_kernel<DD, 4, false>();             \
    default: return qbf16 ? stream_kernel<DD, 8, true>() : stream_kernel<DD, 8, false>();            \
    }
    if (D == 64) { KVQ_SKG(64) }
    if (D == 128) { KVQ_SKG(128) }
    KVQ_SKG(256)
#undef KVQ_SKG
}

// Workgroups of an instantiation that fit on the device at once: per CU the
// smaller of its occupancy target, the VGPR limit (512 per SIMD lane, a
// workgroup puts SNW / 4 waves on each SIMD) and the LDS limit; times the CUs.
static int stream_resident(int D, int G, bool qbf16) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    const int key = ((D == 64 ? 0 : D == 128 ? 1 : 2) * 4 + (G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3)) * 2 +
                    (qbf16 ? 1 : 0);
    static int cache[64][24];                         // 0 = not known yet; benign races
    int v = cache[dev][key];
    if (v > 0) return v;
    hipFuncAttributes fa;
    int cus = 0, lds_cu = 0;
    if (hipFuncGetAttributes(&fa, stream_kernel_for(D, G, qbf16)) != hipSuccess || fa.numRegs <= 0 ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 0;
    if (hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
        lds_cu <= 0)
        lds_cu = 160 * 1024;
    int per_cu = stream_occupancy(G);
    const int by_regs = 512 / ((fa.numRegs + 7) / 8 * 8) / (SNW / 4);   // a workgroup puts SNW / 4 waves on each SIMD
    if (by_regs < per_cu) per_cu = by_regs;
    if (fa.sharedSizeBytes > 0 && lds_cu / (int)fa.sharedSizeBytes < per_cu) per_cu = lds_cu / (int)fa.sharedSizeBytes;
    if (per_cu < 1) per_cu = 1;
    v = per_cu * cus;
    cache[dev][key] = v;
    return v;
}

int stream_splits(int B, int Hkv, int S, int D, int G, bool qbf16) {
    int target = stream_resident(D, G, qbf16);
    if (target <= 0 || target > 3 * 256 * 4 / SNW) target = 2 * 256 * 4 / SNW;
    return splits_for(B, Hkv, S, D, G, target);
}

template <int D, int G, bool QBF16>
static void launch_stream_t(const StreamArgs& a, int nwg, hipStream_t s) {
    hipLaunchKernelGGL((sdpa_decode_stream<D, G, QBF16>), dim3(nwg), dim3(SNT), 0, s, a);
}

template <int D, bool QBF16>
static hipError_t launch_stream_g(const StreamArgs& a, int G, int nwg, hipStream_t s) {
    switch (G) {
    case 1: launch_stream_t<D, 1, QBF16>(a, nwg, s); break;
    case 2: launch_stream_t<D, 2, QBF16>(a, nwg, s); break;
    case 4: launch_stream_t<D, 4, QBF16>(a, nwg, s); break;
    case 8: launch_stream_t<D, 8, QBF16>(a, nwg, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_sdpa_decode_stream(const DecodeLaunch& L, hipStream_t s) {
    const int G = L.Hq / L.Hkv;
    StreamArgs a{L.q, L.B, L.Hq, L.Hkv, L.S, L.kc, L.ks, L.kz, L.vc, L.vs, L.vz, L.kv_len, L.kv_len_sb, L.mask,
                 L.mask_sb, L.sm_scale * 1.4426950408889634f, L.nsplit, L.ctr, L.part_ml, L.part_o, L.out,
                 L.out_bf16 ? 1 : 0, L.err};
    const int nwg = L.B * L.Hkv * L.nsplit;
    switch (L.D) {
    case 64: return L.q_bf16 ? launch_stream_g<64, true>(a, G, nwg, s) : launch_stream_g<64, false>(a, G, nwg, s);
    case 128: return L.q_bf16 ? launch_stream_g<128, true>(a, G, nwg, s) : launch_stream_g<128, false>(a, G, nwg, s);
    case 256: return L.q_bf16 ? launch_stream_g<256, true>(a, G, nwg, s) : launch_stream_g<256, false>(a, G, nwg, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
