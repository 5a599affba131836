// Host interface of the crop and state-copy kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mtp {

hipError_t run_kv_crop(int32_t* len, const int32_t* new_len, int B, hipStream_t st);
hipError_t run_copy_states(void* dst, const void* src, size_t bytes_per_seq, int B, const int32_t* n_accept, int D,
                           hipStream_t st);

}  // namespace mtp
