// One-time weight conversion into the library's layouts (run at weight
// registration, outside the verification step).

#include "common.h"
#include "internal.h"

namespace sv {

__device__ __forceinline__ uint32_t load_bits16(const void* src, int dtype, size_t i) {
  if (dtype == 1) return reinterpret_cast<const uint16_t*>(src)[i];
  return bf16_bits_rne(reinterpret_cast<const float*>(src)[i]);
}

// One thread per 16-byte MFMA chunk (see Mat in internal.h for the layout).
__global__ void k_pack_mfma(const void* src, int dtype, int K, int N, uint4* dst, int KS, int nt,
                            size_t total) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int lane = (int)(idx & 63);
  const size_t rest = idx >> 6;
  const int t = (int)(rest % nt);
  const size_t bs = rest / nt;
  const int s = (int)(bs % KS);
  const int b = (int)(bs / KS);
  const int k0 = s * kKStep + 8 * (lane >> 4);
  const int n = (b * nt + t) * kSub + (lane & 15);
  uint32_t h[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    h[j] = (k0 + j < K && n < N) ? load_bits16(src, dtype, (size_t)(k0 + j) * N + n) : 0u;
  dst[idx] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                        h[6] | (h[7] << 16));
}

// Zero-padded row-major copy, keeping the element type.
__global__ void k_copy_rowmajor(const void* src, int dtype, int K, int N, void* dst, int Kp, int Np) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)Kp * Np) return;
  const int k = (int)(idx / Np), n = (int)(idx - (size_t)k * Np);
  const bool in = k < K && n < N;
  if (dtype == 1) {
    reinterpret_cast<uint16_t*>(dst)[idx] =
        in ? reinterpret_cast<const uint16_t*>(src)[(size_t)k * N + n] : (uint16_t)0;
  } else {
    reinterpret_cast<float*>(dst)[idx] = in ? reinterpret_cast<const float*>(src)[(size_t)k * N + n] : 0.f;
  }
}

__global__ void k_vec_to_f32(const void* src, int dtype, int n, float* dst) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  dst[i] = src == nullptr ? 1.0f
         : dtype == 1 ? bf16_lo(reinterpret_cast<const uint16_t*>(src)[i])
                      : reinterpret_cast<const float*>(src)[i];
}

hipError_t launch_pack_mfma(const void* src, int src_dtype, int K, int N, void* dst, int Kp,
                            int Np, int nt, hipStream_t st) {
  const int KS = Kp / kKStep;
  const size_t total = (size_t)(Np / kSub) * KS * 64;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(k_pack_mfma, dim3(blocks), dim3(256), 0, st, src, src_dtype, K, N,
                     reinterpret_cast<uint4*>(dst), KS, nt, total);
  return hipGetLastError();
}

hipError_t launch_copy_rowmajor(const void* src, int src_dtype, int K, int N, void* dst,
                                int dst_dtype, int Kp, int Np, hipStream_t st) {
  if (src_dtype != dst_dtype) return hipErrorInvalidValue;
  const size_t total = (size_t)Kp * Np;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(k_copy_rowmajor, dim3(blocks), dim3(256), 0, st, src, src_dtype, K, N, dst, Kp, Np);
  return hipGetLastError();
}

hipError_t launch_vec_to_f32(const void* src, int src_dtype, int n, float* dst, hipStream_t st) {
  hipLaunchKernelGGL(k_vec_to_f32, dim3((n + 255) / 256), dim3(256), 0, st, src, src_dtype, n, dst);
  return hipGetLastError();
}

}  // namespace sv
