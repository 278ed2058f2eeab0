// LDS poisoning for debug builds (-DGDN_LDS_POISON).
//
// GDN_LDS_POISON_ALL(a, b, ...) at the top of a kernel, before any return,
// fills the named __shared__ objects with 0xFFFFFFFF words (a NaN as fp32,
// fp16 and bf16; -1 as an int) and waits for the whole workgroup. A result
// computed from LDS that no thread of the workgroup wrote then comes out NaN
// or wrong, and the poisoned build's outputs differ from the normal build's
// (a GPU test compares the two libraries' results). Without GDN_LDS_POISON the
// macro expands to nothing.
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {

template <typename T>
__device__ __forceinline__ void lds_poison_one(T& obj) {
    static_assert(sizeof(T) % 4 == 0, "shared objects are whole 32-bit words");
    unsigned* w = reinterpret_cast<unsigned*>(&obj);
    for (unsigned i = threadIdx.x; i < sizeof(T) / 4; i += blockDim.x) w[i] = 0xFFFFFFFFu;
}

template <typename... T>
__device__ __forceinline__ void lds_poison(T&... objs) {
    (lds_poison_one(objs), ...);
    __syncthreads();
}

}  // namespace gdn

#ifdef GDN_LDS_POISON
#define GDN_LDS_POISON_ALL(...) ::gdn::lds_poison(__VA_ARGS__)
#else
#define GDN_LDS_POISON_ALL(...) ((void)0)
#endif
