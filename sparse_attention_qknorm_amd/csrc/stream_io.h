// Global loads and stores for data a streaming pass touches exactly once.
//
// They carry the nontemporal hint (the `nt` bit of global_load / global_store),
// so the bytes do not compete for cache space with data that is reused. On the
// streaming passes of this library (prologue, pooling, block codecs), whose
// inputs and outputs are far larger than the caches, they are 3-9% faster than
// plain accesses, with the same results.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace saq {

typedef uint32_t u32x4_once __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_once __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_once(const uint4* p) {
    const u32x4_once r = __builtin_nontemporal_load((const u32x4_once*)p);
    return make_uint4(r.x, r.y, r.z, r.w);
}

__device__ __forceinline__ uint2 load_once(const uint2* p) {
    const u32x2_once r = __builtin_nontemporal_load((const u32x2_once*)p);
    return make_uint2(r.x, r.y);
}

__device__ __forceinline__ void store_once(uint4* p, uint4 v) {
    __builtin_nontemporal_store((u32x4_once){v.x, v.y, v.z, v.w}, (u32x4_once*)p);
}

__device__ __forceinline__ void store_once(uint2* p, uint2 v) {
    __builtin_nontemporal_store((u32x2_once){v.x, v.y}, (u32x2_once*)p);
}

}  // namespace saq
