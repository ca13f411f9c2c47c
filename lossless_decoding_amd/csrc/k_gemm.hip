// Projection / FFN / LM-head GEMMs: Y[r][n] = sum_k X[r][k] W[n][k], with
// the small per-row operations of the layer fused into prologue/epilogue.
//
// bf16 path (MFMA v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//  * Operands: the packed weight is the A operand (16 output features x 32
//    k per 1 KB fragment, one coalesced wave load); the activations are the
//    B operand, staged once per workgroup into LDS in fragment order.
//  * Work split: a workgroup owns 128 output columns (8 waves x 16) and up
//    to 64 rows.  K is cut into 8 equal slices.  Each slice is a chain of
//    MFMAs in increasing k starting from zero; the 8 slice sums are added
//    in slice order, ((s0+s1)+s2)+...+s7.  Narrow GEMMs
//    give every slice its own workgroup (8x the workgroups, to stream the
//    weights with the whole chip) and the last workgroup of a column group
//    adds the partials; wide GEMMs keep all slices in one workgroup.  Both
//    produce the same bits, and nothing in the order depends on the number
//    of rows -- a row's output is identical whether computed alone (plain
//    decoding), as the anchor of a draft block or as one of K verify rows.
//  * Prologue: an input that is RMSNorm(h) is normalised while staging
//    (1/rms from per-128-column partial sums of squares, added in order).
//  * Epilogues: QK-norm + RoPE + KV placement (QKV projection; a column
//    group is one head), residual add + partial sums of squares for the
//    next RMSNorm (O and down projections), SwiGLU (gate/up), and per-row
//    argmax with lowest-index ties (LM head; the grid's last workgroup
//    turns the partials into tokens).
//
// fp32 path: one thread per output with a sequential k loop (check models).
#include "internal.h"

#define NSL 8                 // K slices
#define WAVES 8
#define COLS 128              // output columns per workgroup

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ floatx4_t add4(floatx4_t a, floatx4_t b) {
  floatx4_t r;
  r[0] = a[0] + b[0]; r[1] = a[1] + b[1]; r[2] = a[2] + b[2]; r[3] = a[3] + b[3];
  return r;
}

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Coherent (agent-scope) scalar store / load for data read by another
// workgroup of the same launch.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// (value, index) argmax combine: larger value wins, lowest index on ties.
__device__ __forceinline__ void amax_comb(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

template <int MT, int EP, int SPW>
__global__ __launch_bounds__(512, 4) void k_gemm_bf16(GemmArgs a) {
  // LDS: activation block in fragment order (MT*16 rows x 512 k bf16), reused
  // by the epilogue as an fp32 tile of MT*16 x 128.
  __shared__ __attribute__((aligned(16))) uint16_t sX[MT * 16 * 512];
  __shared__ float sInv[64];
  __shared__ float sRed[WAVES * 64];
  __shared__ int sIdx[WAVES * 64];
  __shared__ int sLast;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
  const int KB = a.K >> 5;                   // k-blocks of 32
  const int KS = a.K / NSL;                  // slice length
  const int CL = KS < 256 ? KS : 256;        // k per LDS chunk
  const int CLB = CL >> 5;                   // k-blocks per chunk (<= 8)
  const int ngroups = a.N / COLS;
  int ng, s_first;
  if (SPW == NSL) {
    ng = blockIdx.x; s_first = 0;
  } else if ((ngroups & 7) == 0) {           // keep a column group's slices on one XCD
    const int id = blockIdx.x;
    s_first = (id >> 3) & 7;
    ng = ((id >> 6) << 3) | (id & 7);
  } else {
    s_first = blockIdx.x % NSL;
    ng = blockIdx.x / NSL;
  }
  const int m0 = blockIdx.y * 64;            // GEMM-local first row of this workgroup
  const int nbk = ng * WAVES + wave;         // this wave's 16-column block
  const u32x4_t* wp = a.W + (size_t)nbk * KB * 64 + lane;

  // 1/rms of every row (normalised-input GEMMs): partial sums added in order
  if (a.h && tid < MT * 16) {
    int r = m0 + tid;
    float inv = 0.f;
    if (r < a.M) {
      const float* ss = a.ss + (size_t)(a.row0 + r) * a.nss;
      float t = 0.f;
      for (int j = 0; j < a.nss; ++j) t += ss[j];
      inv = 1.0f / sqrtf(t / (float)a.dn + a.eps);
    }
    sInv[tid] = inv;
  }

  floatx4_t cur[MT], tot[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    cur[mt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    tot[mt] = cur[mt];
  }

  // Weights stream in chunks of CLB k-blocks into two register sets, loaded
  // two chunks ahead; activations are staged into LDS in blocks of SAB
  // k-blocks (up to 512 k), so the weight loads stay in flight across the
  // staging barriers.
  const int nchunk_slice = KS / CL;
  const int nchunks = nchunk_slice * SPW;
  const int kbase0 = s_first * KS;
  const int SAB = (KS >> 5) < 16 ? (KS >> 5) : 16;   // staged k-blocks
  u32x4_t wA[8], wB[8];
  auto wload = [&](u32x4_t (&w)[8], int c) {
    const int kb = (kbase0 >> 5) + c * CLB;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < CLB) w[j] = __builtin_nontemporal_load(wp + (size_t)(kb + j) * 64);
  };
#pragma unroll
  for (int j = 0; j < 8; ++j) { wA[j] = u32x4_t{0u, 0u, 0u, 0u}; wB[j] = wA[j]; }
  wload(wA, 0);
  if (nchunks > 1) wload(wB, 1);

  auto stage = [&](int kb0) {        // stage k-blocks [kb0, kb0 + SAB) of the activations
    __syncthreads();
    const int k0 = kb0 * 32;
    const int units = MT * 16 * SAB * 4;      // 16-byte units
    for (int u = tid; u < units; u += 512) {
      int row = u / (SAB * 4), kq = u - row * (SAB * 4);
      int kb = kq >> 2, q = kq & 3;
      int r = m0 + row;
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (r < a.M) {
        int prw = a.row0 + r;
        if (a.h) {
          const float* hp = a.h + (size_t)prw * a.dn + k0 + kq * 8;
          float4 x0 = *(const float4*)hp, x1 = *(const float4*)(hp + 4);
          uint16_t g[8];
          *(u32x4_t*)g = *(const u32x4_t*)(a.gain + k0 + kq * 8);
          float inv = sInv[row];
          uint16_t e[8];
          e[0] = f2bf(x0.x * inv * bf2f(g[0])); e[1] = f2bf(x0.y * inv * bf2f(g[1]));
          e[2] = f2bf(x0.z * inv * bf2f(g[2])); e[3] = f2bf(x0.w * inv * bf2f(g[3]));
          e[4] = f2bf(x1.x * inv * bf2f(g[4])); e[5] = f2bf(x1.y * inv * bf2f(g[5]));
          e[6] = f2bf(x1.z * inv * bf2f(g[6])); e[7] = f2bf(x1.w * inv * bf2f(g[7]));
          __builtin_memcpy(&v, e, 16);
        } else {
          v = *(const u32x4_t*)(a.X + (size_t)prw * a.ldx + k0 + kq * 8);
        }
      }
      int mt = row >> 4, ln = q * 16 + (row & 15);
      *(u32x4_t*)(sX + ((size_t)(mt * SAB + kb) * 64 + ln) * 8) = v;
    }
    __syncthreads();
  };
  auto compute = [&](const u32x4_t (&w)[8], int c) {
    const int kbl = (c * CLB) % SAB;           // first k-block of the chunk inside the stage
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < CLB) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          u32x4_t xv = *(const u32x4_t*)(sX + ((size_t)(mt * SAB + kbl + j) * 64 + lane) * 8);
          cur[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w[j]), as_bf16x8(xv),
                                                            cur[mt], 0, 0, 0);
        }
      }
    }
    if (SPW == NSL && (c + 1) % nchunk_slice == 0) {   // slice done: add in slice order
      const int s = (c + 1) / nchunk_slice - 1;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        tot[mt] = s == 0 ? cur[mt] : add4(tot[mt], cur[mt]);
        cur[mt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  for (int c = 0; c < nchunks; c += 2) {
    if ((c * CLB) % SAB == 0) stage((kbase0 >> 5) + c * CLB);
    compute(wA, c);
    if (c + 2 < nchunks) wload(wA, c + 2);
    if (c + 1 < nchunks) {
      if (((c + 1) * CLB) % SAB == 0) stage((kbase0 >> 5) + (c + 1) * CLB);
      compute(wB, c + 1);
      if (c + 3 < nchunks) wload(wB, c + 3);
    }
  }
  if (SPW == NSL) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) cur[mt] = tot[mt];
  }

  // ---- split-K: write the slice partial; the last slice workgroup adds all 8.
  // The partials and counters use agent-scope (coherent) stores and loads; an
  // explicit wait for the stores plus the barrier orders them before the
  // counter increment, so no L2 writeback is needed.
  if (SPW == 1) {
    // partial layout [slice][m-group][col group][mt][wave][i][lane]: each
    // coherent dword store of a wave covers 256 contiguous bytes
    const size_t pstride = (size_t)gridDim.y * ngroups * MT * WAVES * 256;
    float* pbase = a.part + ((size_t)blockIdx.y * ngroups + ng) * MT * WAVES * 256;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float* pp = pbase + s_first * pstride + ((size_t)mt * WAVES + wave) * 256 + lane;
#pragma unroll
      for (int i = 0; i < 4; ++i) st_agent(pp + i * 64, cur[mt][i]);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      unsigned* cp = a.cnt + blockIdx.y * ngroups + ng;
      unsigned old = __hip_atomic_fetch_add(cp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sLast = old == NSL - 1;
      if (old == NSL - 1)          // every slice has arrived: reset for the next launch
        __hip_atomic_store(cp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!sLast) return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      floatx4_t p[NSL];
#pragma unroll
      for (int s = 0; s < NSL; ++s) {
        const float* pp = pbase + s * pstride + ((size_t)mt * WAVES + wave) * 256 + lane;
#pragma unroll
        for (int i = 0; i < 4; ++i) p[s][i] = ld_agent(pp + i * 64);
      }
      floatx4_t t = p[0];
#pragma unroll
      for (int s = 1; s < NSL; ++s) t = add4(t, p[s]);
      cur[mt] = t;
    }
  }

  // ============================ epilogues
  // lane (lr, lq) of wave w holds rows m0 + mt*16 + lr, columns nbk*16 + lq*4 + i
  float* tile = (float*)sX;                  // [MT*16][COLS] fp32 scratch
  __syncthreads();
  if (EP == EP_RESID) {
    // h += y; per-row sum of squares of the new values over this column group
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      int r = m0 + mt * 16 + lr;
      float sq = 0.f;
      if (r < a.M) {
        float* yp = a.y + (size_t)(a.row0 + r) * a.ldy + nbk * 16 + lq * 4;
        float4 o = *(float4*)yp;
        o.x += cur[mt][0]; o.y += cur[mt][1]; o.z += cur[mt][2]; o.w += cur[mt][3];
        *(float4*)yp = o;
        sq = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
      }
      sq += __shfl_xor(sq, 16, 64);
      sq += __shfl_xor(sq, 32, 64);
      if (lq == 0) sRed[wave * 64 + mt * 16 + lr] = sq;
    }
    __syncthreads();
    if (tid < MT * 16 && m0 + tid < a.M) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) t += sRed[w * 64 + tid];
      a.ss_out[(size_t)(a.row0 + m0 + tid) * a.nss_out + ng] = t;
    }
    return;
  }
  if (EP == EP_SWIGLU) {
    // odd waves hold the up block of the even wave before them
    if (wave & 1) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        *(floatx4_t*)(tile + ((mt * 16 + lr) * COLS) + (wave >> 1) * 16 + lq * 4) = cur[mt];
    }
    __syncthreads();
    if (!(wave & 1)) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        int r = m0 + mt * 16 + lr;
        if (r >= a.M) continue;
        floatx4_t u = *(const floatx4_t*)(tile + ((mt * 16 + lr) * COLS) + (wave >> 1) * 16 + lq * 4);
        int j = (ng * 4 + (wave >> 1)) * 16 + lq * 4;
        uint16_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = f2bf(silu_f(cur[mt][i]) * u[i]);
        uint2 pk;
        __builtin_memcpy(&pk, o, 8);
        *(uint2*)(a.act + (size_t)(a.row0 + r) * a.ldact + j) = pk;
      }
    }
    return;
  }
  if (EP == EP_ARGMAX) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      int r = m0 + mt * 16 + lr;
      float bv = cur[mt][0];
      int bi = nbk * 16 + lq * 4;
#pragma unroll
      for (int i = 1; i < 4; ++i) amax_comb(bv, bi, cur[mt][i], nbk * 16 + lq * 4 + i);
      if (a.logits && r < a.M)
        *(floatx4_t*)(a.logits + (size_t)(a.row0 + r) * a.ldl + nbk * 16 + lq * 4) = cur[mt];
      float v2 = __shfl_xor(bv, 16, 64); int i2 = __shfl_xor(bi, 16, 64);
      amax_comb(bv, bi, v2, i2);
      v2 = __shfl_xor(bv, 32, 64); i2 = __shfl_xor(bi, 32, 64);
      amax_comb(bv, bi, v2, i2);
      if (lq == 0) { sRed[wave * 64 + mt * 16 + lr] = bv; sIdx[wave * 64 + mt * 16 + lr] = bi; }
    }
    __syncthreads();
    if (tid < MT * 16 && m0 + tid < a.M) {
      float bv = sRed[tid];
      int bi = sIdx[tid];
      for (int w = 1; w < WAVES; ++w) amax_comb(bv, bi, sRed[w * 64 + tid], sIdx[w * 64 + tid]);
      float2* ap = a.amax + (size_t)(a.row0 + m0 + tid) * ngroups + ng;
      st_agent(&ap->x, bv);
      st_agent(&ap->y, __int_as_float(bi));
    }
    // the grid's last surviving workgroup turns the per-group partials into tokens
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      unsigned* cp = a.cnt + gridDim.y * ngroups;
      unsigned old = __hip_atomic_fetch_add(cp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      unsigned total = (unsigned)ngroups * gridDim.y;   // one survivor per column group
      sLast = old == total - 1;
      if (old == total - 1) __hip_atomic_store(cp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!sLast) return;
    for (int r = wave; r < a.M; r += WAVES) {
      const int prow = a.row0 + r;
      const float2* pp = a.amax + (size_t)prow * ngroups;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int j = lane; j < ngroups; j += 64) {
        float tv = ld_agent(&pp[j].x), ti = ld_agent(&pp[j].y);
        amax_comb(bv, bi, tv, __float_as_int(ti));
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        float v2 = __shfl_xor(bv, o, 64); int i2 = __shfl_xor(bi, o, 64);
        amax_comb(bv, bi, v2, i2);
      }
      const PassInfo& P = a.P;
      const RowInfo ri = row_info(P, prow);
      if (lane == 0 && !ri.pad) {
        if (P.kind == PASS_DRAFT) {
          if (!ri.is_mask) {
            if (a.pending) a.pending[ri.b] = bi; else a.ar[(size_t)ri.b * (a.Kb + 1)] = bi;
          } else {
            a.drafts[(size_t)ri.b * a.Kb + (ri.t - P.A)] = bi;
          }
        } else if (P.kind == PASS_VERIFY) {
          a.ar[(size_t)ri.b * (a.Kb + 1) + 1 + ri.t] = bi;
        }
      }
    }
    return;
  }
  if (EP == EP_QKV) {
    // column group ng is one head: q heads, then k heads, then v heads
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *(floatx4_t*)(tile + ((mt * 16 + lr) * COLS) + wave * 16 + lq * 4) = cur[mt];
    __syncthreads();
    const PassInfo& P = a.P;
    const int hd = 128, half = 64;
    const bool isq = ng < a.hq, isk = !isq && ng < a.hq + a.hkv;
    const int head = isq ? ng : (isk ? ng - a.hq : ng - a.hq - a.hkv);
    for (int rl = wave; rl < MT * 16; rl += WAVES) {
      const int r = m0 + rl;
      if (r >= a.M) break;
      const int prow = a.row0 + r;
      const RowInfo ri = row_info(P, prow);
      if (ri.pad || ri.pos >= a.cap) continue;
      float x1 = tile[rl * COLS + lane], x2 = tile[rl * COLS + lane + half];
      float o1 = x1, o2 = x2;
      if (isq || isk) {
        const uint16_t* g = isq ? (ri.is_mask ? a.dqn : a.qn) : (ri.is_mask ? a.dkn : a.kn);
        float ss = wsum(x1 * x1 + x2 * x2);
        float inv = 1.0f / sqrtf(ss / (float)hd + a.eps);
        float y1 = x1 * inv * bf2f(g[lane]), y2 = x2 * inv * bf2f(g[lane + half]);
        float2 cs = a.rope[(size_t)ri.pos * half + lane];
        o1 = y1 * cs.x - y2 * cs.y;
        o2 = y2 * cs.x + y1 * cs.y;
      }
      const int b = ri.b;
      if (isq) {
        uint16_t* qp = a.q_out + (size_t)prow * a.hq * hd + head * hd;
        qp[lane] = f2bf(o1);
        qp[lane + half] = f2bf(o2);
      } else if (ri.is_mask) {
        const int i = ri.t - P.A;
        if (isk) {
          uint16_t* kp = a.ks + (((size_t)b * a.hkv + head) * a.kpad + i) * hd;
          kp[lane] = f2bf(o1);
          kp[lane + half] = f2bf(o2);
        } else {
          uint16_t* vp = a.vs + ((size_t)b * a.hkv + head) * hd * a.kpad;
          const int col = vt_col(i);
          vp[(size_t)lane * a.kpad + col] = f2bf(o1);
          vp[(size_t)(lane + half) * a.kpad + col] = f2bf(o2);
        }
      } else {
        const int p = ri.pos;
        if (isk) {
          uint16_t* kp = a.kc + (((size_t)b * a.hkv + head) * a.cap + p) * hd;
          kp[lane] = f2bf(o1);
          kp[lane + half] = f2bf(o2);
        } else {
          uint16_t* vp = a.vc + (((size_t)b * a.hkv + head) * (a.cap / 64) + p / 64) * (size_t)hd * 64;
          const int col = vt_col(p & 63);
          vp[(size_t)lane * 64 + col] = f2bf(o1);
          vp[(size_t)(lane + half) * 64 + col] = f2bf(o2);
        }
      }
    }
    return;
  }
}

template <int EP, int SPW>
static void dispatch_mt(int MT, dim3 grid, const GemmArgs& a, hipStream_t s) {
  switch (MT) {
    case 1: hipLaunchKernelGGL((k_gemm_bf16<1, EP, SPW>), grid, dim3(512), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_gemm_bf16<2, EP, SPW>), grid, dim3(512), 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_gemm_bf16<3, EP, SPW>), grid, dim3(512), 0, s, a); break;
    default: hipLaunchKernelGGL((k_gemm_bf16<4, EP, SPW>), grid, dim3(512), 0, s, a); break;
  }
}

int gemm_bf16_groups(int N) { return N / COLS; }

void launch_gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0) return;
  const int MT = a.M >= 64 ? 4 : (a.M + 15) / 16;
  const int ng = a.N / COLS;
  bool wide = ng >= 128;                     // enough workgroups without splitting K
  if (a.split == 1) wide = false;
  if (a.split == 2) wide = true;
  dim3 grid(wide ? ng : ng * NSL, (a.M + 63) / 64);
  switch (a.ep) {
    case EP_RESID:
      if (wide) dispatch_mt<EP_RESID, NSL>(MT, grid, a, s); else dispatch_mt<EP_RESID, 1>(MT, grid, a, s);
      break;
    case EP_SWIGLU:
      if (wide) dispatch_mt<EP_SWIGLU, NSL>(MT, grid, a, s); else dispatch_mt<EP_SWIGLU, 1>(MT, grid, a, s);
      break;
    case EP_QKV:
      if (wide) dispatch_mt<EP_QKV, NSL>(MT, grid, a, s); else dispatch_mt<EP_QKV, 1>(MT, grid, a, s);
      break;
    default:
      if (wide) dispatch_mt<EP_ARGMAX, NSL>(MT, grid, a, s); else dispatch_mt<EP_ARGMAX, 1>(MT, grid, a, s);
      break;
  }
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

void launch_gemm_f32(const float* W, const float* W2, const float* X, int ldx, int M, int K,
                     int N, const GemmOut& o, hipStream_t s) {
  if (M <= 0) return;
  dim3 grid((N + 127) / 128, M);
  hipLaunchKernelGGL(k_gemm_f32, grid, dim3(128), 0, s, W, W2, X, ldx, M, K, N, o);
  if (o.ep == EP_ARGMAX)
    hipLaunchKernelGGL(k_argmax_rows_f32, dim3((M + 63) / 64), dim3(64), 0, s, o.y, o.ldy, M, N,
                       o.part);
}
