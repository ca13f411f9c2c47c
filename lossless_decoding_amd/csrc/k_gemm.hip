// Projection / FFN / LM-head GEMMs: Y[r][n] = sum_k X[r][k] W[n][k].
//
// bf16 path (MFMA, gfx950 v_mfma_f32_16x16x32_bf16).  The weight is the A
// operand (16 output features x 32 k), pre-packed so one wave load of 1 KB
// is one fragment; the activations are the B operand (32 k x 16 rows), read
// from row-major bf16 rows.  The reduction order of every output is fixed:
// K is cut into 8 equal slices, each slice is accumulated by a chain of
// MFMAs in increasing k starting from zero, and the 8 slice sums are added
// in slice order.  Nothing in that order depends on how many rows are
// computed together, so a row's output is bit-identical whether it is
// computed alone (plain decoding), as the anchor of a draft block, or as one
// of K verify rows -- which is what makes the draft/verify output identical
// to greedy decoding on the GPU itself.
//
// Workgroup = 8 waves = the 8 K-slices of NB 16-column blocks for up to 64
// rows; the slice partials meet in LDS.  The bound is weight streaming from
// HBM (each weight byte is used by M rows).
//
// fp32 path: one thread per output with a sequential k loop (check models).
#include "internal.h"

#define GEMM_SLICES 8

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

template <int MT, int NB>
__global__ __launch_bounds__(512) void k_gemm_bf16(const u32x4_t* __restrict__ W,
                                                   const uint16_t* __restrict__ X, int ldx,
                                                   int M, int K, GemmOut o) {
  __shared__ float red[GEMM_SLICES * MT * NB * 256];
  const int KB = K >> 5, KBS = KB / GEMM_SLICES;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nb0 = blockIdx.x * NB;
  const int m0 = blockIdx.y * 64;

  floatx4_t acc[MT][NB];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mt][nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const uint16_t* xp[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = m0 + mt * 16 + (lane & 15);
    if (r >= M) r = M - 1;                 // padding rows read a real row; dropped at the end
    xp[mt] = X + (size_t)r * ldx + (lane >> 4) * 8;
  }
  const u32x4_t* wp[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) wp[nb] = W + (size_t)(nb0 + nb) * KB * 64 + lane;

  int kb = wave * KBS;
  const int kend = kb + KBS;
  constexpr int U = 4;
  for (; kb + U <= kend; kb += U) {
    u32x4_t wv[U][NB], xv[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) wv[u][nb] = __builtin_nontemporal_load(wp[nb] + (size_t)(kb + u) * 64);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) xv[u][mt] = *(const u32x4_t*)(xp[mt] + (kb + u) * 32);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mt][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv[u][nb]),
                                                                as_bf16x8(xv[u][mt]),
                                                                acc[mt][nb], 0, 0, 0);
  }
  for (; kb < kend; ++kb) {
    u32x4_t wv[NB], xv[MT];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) wv[nb] = __builtin_nontemporal_load(wp[nb] + (size_t)kb * 64);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xv[mt] = *(const u32x4_t*)(xp[mt] + kb * 32);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[mt][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv[nb]), as_bf16x8(xv[mt]),
                                                              acc[mt][nb], 0, 0, 0);
  }

  // slice partials -> LDS as red[slice][mt][nb][i][lane]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[(((wave * MT + mt) * NB + nb) * 4 + i) * 64 + lane] = acc[mt][nb][i];
  __syncthreads();

  constexpr int E = MT * NB * 256;
  if (o.ep == EP_ARGMAX) {
    // full sums back into slice 0's space, then one thread per row scans
    // its 16*NB columns in increasing order.
    float sums[(E + 511) / 512];
#pragma unroll
    for (int j = 0; j < (E + 511) / 512; ++j) {
      int e = threadIdx.x + j * 512;
      if (e < E) {
        float v = red[e];
#pragma unroll
        for (int s = 1; s < GEMM_SLICES; ++s) v += red[s * E + e];
        sums[j] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < (E + 511) / 512; ++j) {
      int e = threadIdx.x + j * 512;
      if (e < E) {
        red[e] = sums[j];
        if (o.logits) {
          int ln = e & 63, i = (e >> 6) & 3, nb = (e >> 8) % NB, mt = (e >> 8) / NB;
          int row = m0 + mt * 16 + (ln & 15);
          int col = (nb0 + nb) * 16 + (ln >> 4) * 4 + i;
          if (row < M) o.logits[(size_t)row * o.ldl + col] = sums[j];
        }
      }
    }
    __syncthreads();
    if (threadIdx.x < MT * 16) {
      int rl = threadIdx.x, mt = rl >> 4, lr = rl & 15;
      int row = m0 + rl;
      if (row < M) {
        float best = -INFINITY;
        int bidx = -1;
        for (int nb = 0; nb < NB; ++nb)
          for (int q = 0; q < 4; ++q)
            for (int i = 0; i < 4; ++i) {
              float v = red[((mt * NB + nb) * 4 + i) * 64 + q * 16 + lr];
              int col = (nb0 + nb) * 16 + q * 4 + i;
              if (bidx < 0 || v > best) { best = v; bidx = col; }
            }
        o.part[(size_t)row * gridDim.x + blockIdx.x] = make_float2(best, __int_as_float(bidx));
      }
    }
    return;
  }

  for (int e = threadIdx.x; e < E; e += 512) {
    int ln = e & 63, i = (e >> 6) & 3, nb = (e >> 8) % NB, mt = (e >> 8) / NB;
    int row = m0 + mt * 16 + (ln & 15);
    if (row >= M) continue;
    float v = red[e];
#pragma unroll
    for (int s = 1; s < GEMM_SLICES; ++s) v += red[s * E + e];
    int col = (nb0 + nb) * 16 + (ln >> 4) * 4 + i;
    if (o.ep == EP_STORE) {
      o.y[(size_t)row * o.ldy + col] = v;
    } else if (o.ep == EP_RESID) {
      o.y[(size_t)row * o.ldy + col] += v;
    } else if (o.ep == EP_SWIGLU) {
      if (nb & 1) continue;                       // the up half is read by its gate partner
      int e2 = e + 256;                           // same (mt, i, lane), nb + 1
      float u = red[e2];
#pragma unroll
      for (int s = 1; s < GEMM_SLICES; ++s) u += red[s * E + e2];
      int j = ((nb0 + nb) >> 1) * 16 + (ln >> 4) * 4 + i;
      ((uint16_t*)o.act)[(size_t)row * o.ldact + j] = f2bf(silu_f(v) * u);
    }
  }
}

template <int NB>
static void dispatch_mt(int MT, dim3 grid, const void* Wp, const uint16_t* X, int ldx, int M,
                        int K, const GemmOut& o, hipStream_t s) {
  switch (MT) {
    case 1: hipLaunchKernelGGL((k_gemm_bf16<1, NB>), grid, dim3(512), 0, s, (const u32x4_t*)Wp, X, ldx, M, K, o); break;
    case 2: hipLaunchKernelGGL((k_gemm_bf16<2, NB>), grid, dim3(512), 0, s, (const u32x4_t*)Wp, X, ldx, M, K, o); break;
    case 3: hipLaunchKernelGGL((k_gemm_bf16<3, NB>), grid, dim3(512), 0, s, (const u32x4_t*)Wp, X, ldx, M, K, o); break;
    default: hipLaunchKernelGGL((k_gemm_bf16<4, NB>), grid, dim3(512), 0, s, (const u32x4_t*)Wp, X, ldx, M, K, o); break;
  }
}

int gemm_bf16_argmax_parts(int N) { return N / 32; }

void launch_gemm_bf16(const void* Wp, const uint16_t* X, int ldx, int M, int K, int N,
                      const GemmOut& o, hipStream_t s) {
  if (M <= 0) return;
  int MT = M >= 64 ? 4 : (M + 15) / 16;
  int NB = (o.ep == EP_SWIGLU || o.ep == EP_ARGMAX) ? 2 : 1;
  dim3 grid(N / (16 * NB), (M + 63) / 64);
  if (NB == 2) dispatch_mt<2>(MT, grid, Wp, X, ldx, M, K, o, s);
  else dispatch_mt<1>(MT, grid, Wp, X, ldx, M, K, o, s);
}

// ------------------------------------------------------------- fp32
__global__ void k_gemm_f32(const float* __restrict__ W, const float* __restrict__ W2,
                           const float* __restrict__ X, int ldx, int M, int K, int N, GemmOut o) {
  int col = blockIdx.x * blockDim.x + threadIdx.x, row = blockIdx.y;
  if (col >= N || row >= M) return;
  const float* x = X + (size_t)row * ldx;
  const float* w = W + (size_t)col * K;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc += x[k] * w[k];
  if (o.ep == EP_STORE) {
    o.y[(size_t)row * o.ldy + col] = acc;
  } else if (o.ep == EP_RESID) {
    o.y[(size_t)row * o.ldy + col] += acc;
  } else if (o.ep == EP_SWIGLU) {
    const float* w2 = W2 + (size_t)col * K;
    float up = 0.f;
    for (int k = 0; k < K; ++k) up += x[k] * w2[k];
    ((float*)o.act)[(size_t)row * o.ldact + col] = silu_f(acc) * up;
  } else {
    o.y[(size_t)row * o.ldy + col] = acc;       // logits buffer; argmax follows
    if (o.logits) o.logits[(size_t)row * o.ldl + col] = acc;
  }
}

__global__ void k_argmax_rows_f32(const float* __restrict__ lg, int ld, int M, int N,
                                  float2* __restrict__ part) {
  int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= M) return;
  const float* x = lg + (size_t)row * ld;
  float best = x[0];
  int idx = 0;
  for (int j = 1; j < N; ++j)
    if (x[j] > best) { best = x[j]; idx = j; }
  part[row] = make_float2(best, __int_as_float(idx));
}

int gemm_f32_argmax_parts(int N) { (void)N; return 1; }

void launch_gemm_f32(const float* W, const float* W2, const float* X, int ldx, int M, int K,
                     int N, const GemmOut& o, hipStream_t s) {
  if (M <= 0) return;
  dim3 grid((N + 127) / 128, M);
  hipLaunchKernelGGL(k_gemm_f32, grid, dim3(128), 0, s, W, W2, X, ldx, M, K, N, o);
  if (o.ep == EP_ARGMAX)
    hipLaunchKernelGGL(k_argmax_rows_f32, dim3((M + 63) / 64), dim3(64), 0, s, o.y, o.ldy, M, N,
                       o.part);
}
