// Weight packing: rearranges the weights from the notes' x·W layout
// ([in][out] row-major) into the layouts the kernels read (see layout.hpp):
// transposed, concatenated projection rows per branch, fp32 gate factors and
// the stacked transposed output projections.  Runs once per set of weights.
#include "device_common.hpp"
#include "layout.hpp"

namespace msgla {

// dst[c * dst_ld + r] = src[r * Cn + c] for r < R, c < Cn  (transpose of [R][Cn])
template <typename T>
__global__ void k_transpose(const T* __restrict__ src, int R, int Cn, T* __restrict__ dst,
                            size_t dst_ld) {
  __shared__ T tile[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 256 threads: 32 x 8
  for (int k = ty; k < 32; k += 8) {
    const int r = r0 + k, c = c0 + tx;
    if (r < R && c < Cn) tile[k][tx] = src[(size_t)r * Cn + c];
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int c = c0 + k, r = r0 + tx;
    if (r < R && c < Cn) dst[(size_t)c * dst_ld + r] = tile[tx][k];
  }
}

template <typename T>
__global__ void k_to_f32(const T* __restrict__ src, size_t n, float* __restrict__ dst) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = to_f32(src[i]);
}

__global__ void k_fill_zero(uint32_t* __restrict__ p, size_t n_words) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_words) p[i] = 0u;
}

template <typename T>
static hipError_t transpose_into(const void* src, int R, int Cn, void* dst, size_t dst_ld,
                                 hipStream_t st) {
  if (R <= 0 || Cn <= 0) return hipSuccess;
  const dim3 grid((Cn + 31) / 32, (R + 31) / 32);
  hipLaunchKernelGGL(k_transpose<T>, grid, dim3(256), 0, st, reinterpret_cast<const T*>(src), R,
                     Cn, reinterpret_cast<T*>(dst), dst_ld);
  return hipGetLastError();
}

hipError_t pack_transpose(bool bf16_path, const void* src, int R, int Cn, void* dst,
                          size_t dst_ld, hipStream_t st) {
  return bf16_path ? transpose_into<bf16>(src, R, Cn, dst, dst_ld, st)
                   : transpose_into<float>(src, R, Cn, dst, dst_ld, st);
}

hipError_t pack_to_f32(bool src_bf16, const void* src, size_t n, float* dst, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (src_bf16)
    hipLaunchKernelGGL(k_to_f32<bf16>, grid, dim3(256), 0, st, reinterpret_cast<const bf16*>(src),
                       n, dst);
  else
    hipLaunchKernelGGL(k_to_f32<float>, grid, dim3(256), 0, st,
                       reinterpret_cast<const float*>(src), n, dst);
  return hipGetLastError();
}

hipError_t fill_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace msgla
