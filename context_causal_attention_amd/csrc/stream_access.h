// Streaming global accesses for the bandwidth-bound kernels (reorder, permute, merge, delta).
// Their data is read once and written once, so 16-byte accesses go non-temporal: kept out of
// the caches, a 512 MiB copy measured 6.4 TB/s against 5.1 TB/s with cached accesses, with
// one 16-byte access per lane and many small blocks (more accesses per lane measured lower).
// Other element types are accessed normally.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <typename T>
__device__ inline T load_stream(const T* p) { return *p; }
template <typename T>
__device__ inline void store_stream(T* p, const T& v) { *p = v; }

template <>
__device__ inline v4u load_stream<v4u>(const v4u* p) { return __builtin_nontemporal_load(p); }
template <>
__device__ inline void store_stream<v4u>(v4u* p, const v4u& v) { __builtin_nontemporal_store(v, p); }
template <>
__device__ inline v4f load_stream<v4f>(const v4f* p) { return __builtin_nontemporal_load(p); }
template <>
__device__ inline void store_stream<v4f>(v4f* p, const v4f& v) { __builtin_nontemporal_store(v, p); }

}  // namespace cpattn
