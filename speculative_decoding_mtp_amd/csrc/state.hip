// KV-cache crop and recurrent-state snapshot / masked restore.
//
// [HB14] "14. MTP: speculative decoding with the built-in draft head", section "The draft head":
// rolling an attention cache back keeps its first n positions; a recurrent memory table cannot
// be truncated, so it is copied before verification and copied back on a miss.  [DLM] "The
// decoding loop and MTP", item 2: the cache is cut back after the first refused guess.
#include "common.h"
#include "state.h"

namespace mtp {

// len[b] = min(len[b], max(new_len[b], 0))
__global__ void k_kv_crop(int32_t* len, const int32_t* new_len, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) {
    const int n = max(new_len[b], 0);
    if (n < len[b]) len[b] = n;
  }
}

// dst[b] = src[b] for the sequences selected by mask (all when n_accept is NULL); grid.y =
// sequence, grid.x sized so that four strides of the grid cover a sequence: each thread has its
// four 16-byte loads in flight at once (unconditional, from clamped addresses), then stores the
// ones inside the sequence.
__global__ __launch_bounds__(kWG) void k_copy_states(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                     long vec_per_seq, const int32_t* n_accept, int D) {
  const int b = blockIdx.y;
  if (n_accept && n_accept[b] >= D) return;
  const uint4* s = src + (long)b * vec_per_seq;
  uint4* d = dst + (long)b * vec_per_seq;
  const long stride = (long)gridDim.x * kWG;
  const long i = (long)blockIdx.x * kWG + threadIdx.x;
  uint4 a[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) a[k] = ld_stream(s + min(i + k * stride, vec_per_seq - 1));
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (i + k * stride < vec_per_seq)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&a[k]), reinterpret_cast<u32x4*>(d + i + k * stride));
}

hipError_t run_kv_crop(int32_t* len, const int32_t* new_len, int B, hipStream_t st) {
  hipLaunchKernelGGL(k_kv_crop, dim3((B + kWG - 1) / kWG), dim3(kWG), 0, st, len, new_len, B);
  return hipGetLastError();
}

hipError_t run_copy_states(void* dst, const void* src, size_t bytes_per_seq, int B, const int32_t* n_accept, int D,
                           hipStream_t st) {
  const long vec = (long)(bytes_per_seq / 16);
  // 16 KB of a sequence per workgroup (four 16-byte vectors per thread)
  const long per_seq = (vec + 4 * kWG - 1) / (4 * kWG);
  if (per_seq > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_copy_states, dim3((unsigned)per_seq, B), dim3(kWG), 0, st, reinterpret_cast<uint4*>(dst),
                     reinterpret_cast<const uint4*>(src), vec, n_accept, D);
  return hipGetLastError();
}

}  // namespace mtp
