// Buffer-resource and global->LDS copy helpers for gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

// Raw buffer resource over [base, base + bytes): loads at offsets past the
// range return zeros (no fault, no branch). The range is clamped to 2^31 - 1.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t lim = bytes < 0 ? 0 : (bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(lim),
                                           0x00020000);
}

// LDS pointer type of the global->LDS buffer loads
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace qlora
