// Device fill for seeded synthetic inputs: the same Philox4x32-10
// (Salmon et al., SC'11) and value maps as synth/__init__.py, written
// straight into device memory so multi-GB random-init models need no host
// round trip.  No arithmetic of the decoding method lives here.
#include <hip/hip_runtime.h>
#include <stdint.h>

__device__ __forceinline__ void philox10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
    uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
    uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
  }
}

__global__ void k_fill_normal(void* out, uint64_t n, uint64_t start, uint64_t seed,
                              uint32_t stream, uint32_t purpose, float scale, int kind) {
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) {
    uint64_t e = start + i;
    uint32_t c[4] = {(uint32_t)e, (uint32_t)(e >> 32), stream, purpose};
    philox10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    int32_t s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) s += (int32_t)(c[j] & 0xFFFFu) + (int32_t)(c[j] >> 16);
    float v = __fmul_rn((float)(s - 262140), scale);
    if (kind == 0) {
      ((float*)out)[i] = v;
    } else {
      uint32_t u = __float_as_uint(v);
      uint32_t rnd = ((u >> 16) & 1u) + 0x7FFFu;
      ((uint16_t*)out)[i] = (uint16_t)((u + rnd) >> 16);
    }
  }
}

__global__ void k_fill_const(void* out, uint64_t n, float v, int kind) {
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint32_t u = __float_as_uint(v);
  uint16_t b = (uint16_t)((u + ((u >> 16) & 1u) + 0x7FFFu) >> 16);
  for (; i < n; i += stride) {
    if (kind == 0) ((float*)out)[i] = v; else ((uint16_t*)out)[i] = b;
  }
}

static unsigned grid_for(uint64_t n) {
  uint64_t g = (n + 255) / 256;
  return (unsigned)(g > 65536 ? 65536 : (g ? g : 1));
}

extern "C" int synth_dev_fill_normal(void* out, uint64_t n, uint64_t start, uint64_t seed,
                                     uint32_t stream, uint32_t purpose, float scale, int kind,
                                     void* hstream) {
  if (!out || n == 0) return n == 0 ? 0 : -1;
  hipLaunchKernelGGL(k_fill_normal, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)hstream, out,
                     n, start, seed, stream, purpose, scale, kind);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int synth_dev_fill_const(void* out, uint64_t n, float v, int kind, void* hstream) {
  if (!out || n == 0) return n == 0 ? 0 : -1;
  hipLaunchKernelGGL(k_fill_const, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)hstream, out, n,
                     v, kind);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
