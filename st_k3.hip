#include <hip/hip_runtime.h>
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));
namespace d {
template <int N> __global__ void k1(const u4* g, float* o) {
  __shared__ __attribute__((aligned(16))) u4 s[64];
  __builtin_amdgcn_global_load_lds(g + threadIdx.x, s, 16, 0, 0);
  __syncthreads();
  o[threadIdx.x] = (float)s[threadIdx.x][0] + N;
}
template <int N> __global__ void k2(const u4* g, float* o) {
  __shared__ __bf16 s[256];
  bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(s + 4 * threadIdx.x));
  o[threadIdx.x] = (float)v[0] + N;
}
template <int N> __global__ void k3(const u4* g, float* o) {
  if (__builtin_amdgcn_ballot_w64(o[threadIdx.x] > 0)) o[threadIdx.x] = N;
}
template <int N> __global__ void k4(const u4* g, float* o) {
  __builtin_amdgcn_s_waitcnt(0xF70);
  o[threadIdx.x] = N;
}
}
void launch(const u4* g, float* o) { hipLaunchKernelGGL(d::k3<1>, dim3(1), dim3(64), 0, 0, g, o); }
