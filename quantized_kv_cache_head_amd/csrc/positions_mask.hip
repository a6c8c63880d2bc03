// positions_mask.hip -- slot positions for full / ring / sink caches and the
// additive mask of ring and sink caches.
//
// pytorch/executorch PR 24473, Summary: a sink cache pins sink_size slots and
// runs the remaining window slots as a ring (slots from the positions manager
// with sink); a ring cache is the same with sink_size 0; a full-context cache
// writes position p to slot p and rejects a write past its slot count; ring
// and sink caches attend with an additive float mask built from the position
// each slot holds.
//
// The start position is a device scalar so the step can be replayed without
// host involvement; one thread per token / per mask element.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

// sink_size >= 0, window >= 1.  Thread t handles position p = start + t.
// Within one call a later position overwrites an earlier one in the same
// slot; only the last writer of each slot stores cache_positions, so the
// result does not depend on thread order.
__global__ __launch_bounds__(256) void positions_sink_kernel(const int32_t* start_pos, int T, int sink,
                                                             int window, int32_t* slot_out,
                                                             int32_t* cache_positions, int32_t* err) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    const int start = *start_pos;
    if (start < 0) {
        slot_out[t] = -1;
        if (t == 0 && err) atomicOr(err, KVQ_DEV_FLAG_SLOT_RANGE);
        return;
    }
    const int64_t p = (int64_t)start + t;
    int slot;
    if (p < sink) slot = (int)p;
    else slot = sink + (int)((p - sink) % window);
    // a token whose slot a later token of the same call takes again is not
    // written (slot -1): the cache then holds what writing the tokens one
    // after another leaves, and one call never scatters to a slot twice
    const int64_t last = (int64_t)start + T - 1;
    const bool last_writer = p < sink || p + window > last;
    slot_out[t] = last_writer ? slot : -1;
    if (cache_positions && last_writer) cache_positions[slot] = (int32_t)p;
}

__global__ __launch_bounds__(256) void positions_full_kernel(const int32_t* start_pos, int T, int capacity,
                                                             int32_t* slot_out, int32_t* cache_positions,
                                                             int32_t* err) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    const int start = *start_pos;
    const int64_t p = (int64_t)start + t;
    if (start < 0) {
        slot_out[t] = -1;
        if (t == 0 && err) atomicOr(err, KVQ_DEV_FLAG_SLOT_RANGE);
        return;
    }
    if (p >= capacity) {
        slot_out[t] = -1;
        if (err) atomicOr(err, KVQ_DEV_FLAG_POS_CAPACITY);
        return;
    }
    slot_out[t] = (int32_t)p;
    if (cache_positions) cache_positions[p] = (int32_t)p;
}

// mask[r, s] = 0 if cp = cache_positions[s] is visible from qp = start + r:
// cp >= 0, cp <= qp and (cp < sink or qp - cp < window); else -inf.
__global__ __launch_bounds__(256) void build_mask_kernel(const int32_t* cache_positions, int n_slots,
                                                         const int32_t* start_pos, int Lq, int sink,
                                                         int window, float* mask) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)Lq * n_slots) return;
    const int r = (int)(i / n_slots);
    const int s = (int)(i % n_slots);
    const int64_t qp = (int64_t)(*start_pos) + r;
    const int64_t cp = cache_positions[s];
    const bool visible = cp >= 0 && cp <= qp && (cp < sink || qp - cp < window);
    mask[i] = visible ? 0.0f : -__builtin_huge_valf();
}

hipError_t launch_positions_sink(const int32_t* start_pos, int T, int sink, int window, int32_t* slot_out,
                                 int32_t* cache_positions, int32_t* err, hipStream_t s) {
    hipLaunchKernelGGL(positions_sink_kernel, dim3((T + 255) / 256), dim3(256), 0, s, start_pos, T, sink,
                       window, slot_out, cache_positions, err);
    return hipGetLastError();
}

hipError_t launch_positions_full(const int32_t* start_pos, int T, int capacity, int32_t* slot_out,
                                 int32_t* cache_positions, int32_t* err, hipStream_t s) {
    hipLaunchKernelGGL(positions_full_kernel, dim3((T + 255) / 256), dim3(256), 0, s, start_pos, T, capacity,
                       slot_out, cache_positions, err);
    return hipGetLastError();
}

hipError_t launch_build_mask(const int32_t* cache_positions, int n_slots, const int32_t* start_pos, int Lq,
                             int sink, int window, float* mask, hipStream_t s) {
    const int64_t n = (int64_t)Lq * n_slots;
    hipLaunchKernelGGL(build_mask_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, cache_positions,
                       n_slots, start_pos, Lq, sink, window, mask);
    return hipGetLastError();
}

}  // namespace kvq
