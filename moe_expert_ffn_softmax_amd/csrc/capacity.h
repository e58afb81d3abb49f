// Capacity-aware routing (the adaptive token dropper): launcher shared by the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace afd {

// Largest batch: a token's place in its expert's list is kept in 21 bits.
constexpr int kCapMaxTokens = 1 << 21;

// One workgroup walks the T preference lists ids/gates [T,k] in token order (the
// dropper is sequential by definition: each decision reads the counts left by the
// tokens before it).  limits [E] is read and, when `adaptive`, updated in place;
// assign [T], weight [T], offsets [E+1] and sorted_token [T] are written.  E <= 1024,
// k <= 32.
hipError_t launch_route_capacity(const int32_t* ids, const float* gates, int T, int E, int k, int32_t base,
                                 int adaptive, int32_t* limits, int32_t* assign, float* weight, int32_t* offsets,
                                 int32_t* sorted_token, hipStream_t st);

// Fills a route (ids, gates, counts, offsets, sorted_pair, pair_pos for T tokens of k
// slots) from a capacity result so that the expert FFN runs each kept token through
// its one expert with its weight (slot 0) and nothing else.
hipError_t launch_route_from_capacity(const int32_t* assign, const float* weight, const int32_t* cap_offsets,
                                      const int32_t* sorted_token, int T, int E, int k, int32_t* ids, float* gates,
                                      int32_t* counts, int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                                      hipStream_t st);

}  // namespace afd
