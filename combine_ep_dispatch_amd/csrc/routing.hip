// Conversions between compact top-k routing (ids and probabilities [T, K])
// and the dense form (a multihot routing map and probabilities [T, E]).
// NeMo AutoModel token_dispatcher page: _HybridEPManager._indices_to_multihot
// turns indices into a multihot map; NeMo AutoModel fused_a2a page:
// HybridEPDispatch.forward takes either form, the dense map taking
// precedence.
//
// Both kernels use one wave64 per token and walk the experts in chunks of 64
// (lane l owns expert 64*c + l of chunk c), so every map byte and dense
// probability is written by exactly one lane, in one pass, without atomics.
//  - indices -> multihot: each lane compares its expert with the token's K
//    slots (broadcast from lanes 0..K-1 with v_readlane) in slot order, so an
//    expert named twice is set once and its probabilities add in slot order.
//  - multihot -> indices: a ballot of the chunk's marked experts gives each
//    marked lane its slot (running count + rank below it), so slots fill in
//    ascending expert order; lanes past the last used slot write -1 / 0.
//    A row marking more than K experts keeps the lowest K and raises
//    EP_FLAG_MAP_OVERFLOW in the caller's flags word.
#include "epx_device.h"

namespace epx {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / kWave;

__global__ __launch_bounds__(kRouteThreads) void k_indices_to_multihot(RouteArgs a) {
    const int32_t t = uniform((int32_t)(blockIdx.x * kRouteWaves + threadIdx.x / kWave));
    if (t >= a.T) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t my_id = lane < a.K ? a.ids[(int64_t)t * a.K + lane] : -1;
    const float my_p = (lane < a.K && a.probs != nullptr) ? a.probs[(int64_t)t * a.K + lane] : 0.0f;
    for (int32_t e0 = 0; e0 < a.E; e0 += kWave) {
        const int32_t e = e0 + lane;
        uint32_t set = 0;
        float p = 0.0f;
        for (int32_t k = 0; k < a.K; ++k) {
            const int32_t id = __builtin_amdgcn_readlane(my_id, k);
            if (id == e) {
                set = 1;
                p = p + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_p), k));
            }
        }
        if (e < a.E) {
            a.map[(int64_t)t * a.E + e] = (uint8_t)set;
            if (a.dense_probs != nullptr) a.dense_probs[(int64_t)t * a.E + e] = p;
        }
    }
}

__global__ __launch_bounds__(kRouteThreads) void k_multihot_to_indices(RouteArgs a) {
    const int32_t t = uniform((int32_t)(blockIdx.x * kRouteWaves + threadIdx.x / kWave));
    if (t >= a.T) return;
    const int lane = threadIdx.x & (kWave - 1);
    int32_t n = 0;  // marked experts seen so far (wave-uniform)
    for (int32_t e0 = 0; e0 < a.E; e0 += kWave) {
        const int32_t e = e0 + lane;
        const bool marked = e < a.E && a.map[(int64_t)t * a.E + e] != 0;
        const uint64_t m = __builtin_amdgcn_ballot_w64(marked);
        const int32_t slot = n + (int32_t)lanes_below(m);
        if (marked && slot < a.K) {
            a.ids[(int64_t)t * a.K + slot] = e;
            if (a.probs != nullptr) a.probs[(int64_t)t * a.K + slot] = a.dense_probs[(int64_t)t * a.E + e];
        }
        n += (int32_t)__popcll(m);
    }
    if (lane >= n && lane < a.K) {
        a.ids[(int64_t)t * a.K + lane] = -1;
        if (a.probs != nullptr) a.probs[(int64_t)t * a.K + lane] = 0.0f;
    }
    if (n > a.K && lane == 0 && a.flags != nullptr) atomicOr(a.flags, EP_FLAG_MAP_OVERFLOW);
}

}  // namespace

hipError_t launch_indices_to_multihot(const RouteArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((a.T + kRouteWaves - 1) / kRouteWaves);
    hipLaunchKernelGGL(k_indices_to_multihot, dim3(blocks), dim3(kRouteThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_multihot_to_indices(const RouteArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((a.T + kRouteWaves - 1) / kRouteWaves);
    hipLaunchKernelGGL(k_multihot_to_indices, dim3(blocks), dim3(kRouteThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace epx
