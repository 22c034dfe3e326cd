#include <hip/hip_runtime.h>
__global__ void k(const float4* g, float4* o) {
  __shared__ float4 s[256];
  float4 x = g[threadIdx.x + 1024];          // a global load left in flight
  s[threadIdx.x] = g[threadIdx.x];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  float4 y = s[(threadIdx.x + 1) & 255];
  o[threadIdx.x] = make_float4(x.x + y.x, x.y, y.z, y.w);
}
