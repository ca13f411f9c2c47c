// Small kernels of the decode step: weight packing, embedding, RMSNorm,
// QK-norm + RoPE + KV placement, LM-head argmax reduction, acceptance and
// commit.  All reductions run in a fixed order that does not depend on the
// number of rows, so a row's result is the same in every pass.
#include "internal.h"

// ------------------------------------------------------------- packing
// Weight [N][K] bf16 row-major -> MFMA A-operand blocks: block (nb, kb)
// holds rows nb*16..+16, columns kb*32..+32; lane l's 16 bytes are row
// nb*16 + l%16, columns kb*32 + (l/16)*8 .. +8.  Destination block index
// (nb_off + nb*nb_stride, kb) lets gate/up be interleaved per 16 rows.
__global__ void k_pack_bf16(const uint4* __restrict__ src, int N, int K, uint4* __restrict__ dst,
                            int nb_off, int nb_stride) {
  const int KB = K / 32;
  const size_t total = (size_t)(N / 16) * KB * 64;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    int lane = (int)(idx & 63);
    size_t blk = idx >> 6;
    int kb = (int)(blk % KB);
    int nb = (int)(blk / KB);
    int row = nb * 16 + (lane & 15);
    int col = kb * 32 + (lane >> 4) * 8;
    uint4 v = src[((size_t)row * K + col) / 8];
    dst[((size_t)(nb_off + (size_t)nb * nb_stride) * KB + kb) * 64 + lane] = v;
  }
}

void launch_pack_bf16(const uint16_t* src, int N, int K, void* dst, int nb_off, int nb_stride,
                      hipStream_t s) {
  size_t total = (size_t)(N / 16) * (K / 32) * 64;
  unsigned grid = (unsigned)((total + 255) / 256);
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(k_pack_bf16, dim3(grid), dim3(256), 0, s, (const uint4*)src, N, K,
                     (uint4*)dst, nb_off, nb_stride);
}

// ----------------------------------------------------------- embedding
// h[row] = E[token] (token rows) or the mask embedding (mask rows; in a
// refining draft pass the embedding of the row's current draft); padding
// rows get zeros.
__global__ __launch_bounds__(256) void k_embed(PassInfo P, const int32_t* __restrict__ anchor_tok,
                                               const int32_t* __restrict__ block_tok, int block_ld,
                                               const void* __restrict__ embed,
                                               const void* __restrict__ mask_emb, int V, int d,
                                               int bf16, float* __restrict__ h) {
  const int r = blockIdx.x;
  int kind;          // 0 token, 1 mask, 2 padding
  int tok = 0;
  if (P.kind == PASS_DRAFT) {
    if (r >= P.RM) { kind = 0; tok = anchor_tok[r - P.RM]; }
    else if (r < P.B * P.Kx) {
      kind = 1;
      if (P.refine) {                   // the mask row takes its current draft's embedding
        const int b = r / P.Kx;
        kind = 0;
        tok = block_tok[(size_t)b * block_ld + (r - b * P.Kx)];
      }
    } else kind = 2;
  } else {
    int b = r / P.Kx, i = r - b * P.Kx;
    kind = 0;
    tok = block_tok[(size_t)b * block_ld + (P.kind == PASS_PREFILL ? P.p0 : 0) + i];
  }
  tok = tok < 0 ? 0 : (tok >= V ? V - 1 : tok);
  float* out = h + (size_t)r * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    float v = 0.f;
    if (kind != 2) {
      if (bf16) {
        const uint16_t* src = kind == 1 ? (const uint16_t*)mask_emb
                                        : (const uint16_t*)embed + (size_t)tok * d;
        v = bf2f(src[i]);
      } else {
        const float* src = kind == 1 ? (const float*)mask_emb : (const float*)embed + (size_t)tok * d;
        v = src[i];
      }
    }
    out[i] = v;
  }
}

void launch_embed(const PassInfo& P, const int32_t* anchor_tok, const int32_t* block_tok,
                  int block_ld, const void* embed, const void* mask_emb, int V, int d, bool bf16,
                  float* h, hipStream_t s) {
  int rows = P.rows();
  if (rows <= 0) return;
  hipLaunchKernelGGL(k_embed, dim3(rows), dim3(256), 0, s, P, anchor_tok, block_tok, block_ld,
                     embed, mask_emb, V, d, (int)bf16, h);
}

// Residual add of the split-K partials + RMSNorm -> bf16 rows (fragment
// order, the GEMMs' input layout).  One block
// of NW waves per row; the row is cut into 256-element chunks, wave w takes
// chunks w, w + NW, ..., lane l holds elements 4l .. 4l + 3.  All loads are
// issued before use.  The partial sum runs in slice order and is then added
// to h (the same arithmetic as a fused residual epilogue).  The sum of
// squares is canonical: per chunk, the lane's four squares in order and a
// fixed butterfly, then the chunk sums in chunk order, whatever NW is.
template <int NCW, int NW>
__global__ __launch_bounds__(NW * 64) void k_resid_norm_bf16(PassInfo P, float* __restrict__ h, int d,
                                                             const float* __restrict__ part, size_t ps,
                                                             int nslices,
                                                             const uint16_t* __restrict__ gain,
                                                             float eps, uint16_t* __restrict__ out) {
  __shared__ float red[32];
  const int r = blockIdx.x, t = threadIdx.x, wave = t >> 6, lane = t & 63, nch = d >> 8;
  if (P.kind == PASS_DRAFT && row_info(P, r).pad) {     // keep padding rows' input at zero
    for (int i = t * 4; i < d; i += NW * 256) *(uint2*)(out + frag_off(r, i, d >> 5)) = make_uint2(0u, 0u);
    return;
  }
  float* x = h + (size_t)r * d;
  float4 v[NCW];
#pragma unroll
  for (int j = 0; j < NCW; ++j) {
    const int c = wave + j * NW;
    v[j] = c < nch ? *(const float4*)(x + c * 256 + lane * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (nslices == 8) {
    float4 p[8][NCW];
#pragma unroll
    for (int sl = 0; sl < 8; ++sl)
#pragma unroll
      for (int j = 0; j < NCW; ++j) {
        const int c = wave + j * NW;
        p[sl][j] = c < nch ? *(const float4*)(part + sl * ps + (size_t)r * d + c * 256 + lane * 4)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
    for (int j = 0; j < NCW; ++j) {
      float4 s4 = p[0][j];
#pragma unroll
      for (int sl = 1; sl < 8; ++sl) {
        s4.x += p[sl][j].x; s4.y += p[sl][j].y; s4.z += p[sl][j].z; s4.w += p[sl][j].w;
      }
      v[j].x += s4.x; v[j].y += s4.y; v[j].z += s4.z; v[j].w += s4.w;
      const int c = wave + j * NW;
      if (c < nch) *(float4*)(x + c * 256 + lane * 4) = v[j];
    }
  }
#pragma unroll
  for (int j = 0; j < NCW; ++j) {
    const int c = wave + j * NW;
    float sq = v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
    if (c < nch && lane == 0) red[c] = sq;
  }
  __syncthreads();
  float tot = red[0];
  for (int c = 1; c < nch; ++c) tot += red[c];
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int j = 0; j < NCW; ++j) {
    const int c = wave + j * NW, i = c * 256 + lane * 4;
    if (c < nch) {
      const uint2 g = *(const uint2*)(gain + i);
      const float g0 = __uint_as_float(g.x << 16), g1 = __uint_as_float(g.x & 0xffff0000u);
      const float g2 = __uint_as_float(g.y << 16), g3 = __uint_as_float(g.y & 0xffff0000u);
      uint2 o;
      o.x = (uint32_t)f2bf(v[j].x * inv * g0) | ((uint32_t)f2bf(v[j].y * inv * g1) << 16);
      o.y = (uint32_t)f2bf(v[j].z * inv * g2) | ((uint32_t)f2bf(v[j].w * inv * g3) << 16);
      *(uint2*)(out + frag_off(r, i, d >> 5)) = o;
    }
  }
}

// d a multiple of 256, at most 8192: one 256-element chunk per wave up to
// d = 4096 (16 waves), else 16 waves with two chunks each
void launch_resid_norm_bf16(const PassInfo& P, float* h, int d, const float* part, size_t ps,
                            int nslices, const uint16_t* gain, float eps, uint16_t* out,
                            hipStream_t s) {
  const int rows = P.rows();
  if (rows <= 0) return;
  if ((d >> 8) <= 16)
    hipLaunchKernelGGL((k_resid_norm_bf16<1, 16>), dim3(rows), dim3(1024), 0, s, P, h, d, part, ps, nslices, gain, eps, out);
  else
    hipLaunchKernelGGL((k_resid_norm_bf16<2, 16>), dim3(rows), dim3(1024), 0, s, P, h, d, part, ps, nslices, gain, eps, out);
}

// -------------------------------------------------------------- RMSNorm
// One 256-thread block per row.  Thread t sums x[t], x[t+256], ... in order;
// the 256 partials are combined by a fixed binary tree.
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ h, int d,
                                                 const void* __restrict__ gain, int bf16,
                                                 float eps, void* __restrict__ out) {
  __shared__ float red[256];
  int r = blockIdx.x;
  const float* x = h + (size_t)r * d;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) ss += x[i] * x[i];
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  float inv = 1.0f / sqrtf(red[0] / (float)d + eps);
  for (int i = threadIdx.x; i < d; i += 256) {
    if (bf16) {
      float g = bf2f(((const uint16_t*)gain)[i]);
      ((uint16_t*)out)[(size_t)r * d + i] = f2bf(x[i] * inv * g);
    } else {
      float g = ((const float*)gain)[i];
      ((float*)out)[(size_t)r * d + i] = x[i] * inv * g;
    }
  }
}

void launch_rmsnorm(const float* h, int rows, int d, const void* gain, bool bf16, float eps,
                    void* out, hipStream_t s) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(k_rmsnorm, dim3(rows), dim3(256), 0, s, h, d, gain, (int)bf16, eps, out);
}

// ---------------------------------------------- QK-norm + RoPE + KV write
// One wave per (row, head slot): slots [0, hq) are query heads, [hq, hq+hkv)
// KV heads.  Lane i < hd/2 owns the rotate-half pair (i, i + hd/2).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__global__ __launch_bounds__(64) void k_qkv_post(
    PassInfo P, const float* __restrict__ qkv, int hq, int hkv, int hd,
    const void* __restrict__ qn, const void* __restrict__ kn, const void* __restrict__ dqn,
    const void* __restrict__ dkn, int bf16, float eps, const float2* __restrict__ rope,
    void* __restrict__ q_out, void* __restrict__ kc, void* __restrict__ vc, int cap,
    void* __restrict__ ks, void* __restrict__ vs, int kpad) {
  const int r = blockIdx.x, slot = blockIdx.y, lane = threadIdx.x;
  const RowInfo ri = row_info(P, r);
  if (ri.pad || ri.pos >= cap) return;     // padding row, or past the cache (host bound excludes it)
  const int qd = hq * hd, kd = hkv * hd, half = hd / 2;
  const bool isq = slot < hq;
  const int head = isq ? slot : slot - hq;
  const float* src = qkv + (size_t)r * (qd + 2 * kd) + (isq ? head * hd : qd + head * hd);
  const void* gsrc = isq ? (ri.is_mask ? dqn : qn) : (ri.is_mask ? dkn : kn);
  float x1 = 0.f, x2 = 0.f;
  if (lane < half) { x1 = src[lane]; x2 = src[lane + half]; }
  float ss = wave_sum(x1 * x1 + x2 * x2);
  float inv = 1.0f / sqrtf(ss / (float)hd + eps);
  float o1 = 0.f, o2 = 0.f;
  if (lane < half) {
    float g1 = bf16 ? bf2f(((const uint16_t*)gsrc)[lane]) : ((const float*)gsrc)[lane];
    float g2 = bf16 ? bf2f(((const uint16_t*)gsrc)[lane + half])
                    : ((const float*)gsrc)[lane + half];
    float y1 = x1 * inv * g1, y2 = x2 * inv * g2;
    float2 cs = rope[(size_t)ri.pos * half + lane];
    o1 = y1 * cs.x - y2 * cs.y;
    o2 = y2 * cs.x + y1 * cs.y;
  }
  if (lane >= half) return;
  if (isq) {
    size_t base = (size_t)r * qd + (size_t)head * hd;
    if (bf16) {
      ((uint16_t*)q_out)[base + lane] = f2bf(o1);
      ((uint16_t*)q_out)[base + lane + half] = f2bf(o2);
    } else {
      ((float*)q_out)[base + lane] = o1;
      ((float*)q_out)[base + lane + half] = o2;
    }
    return;
  }
  // K and V of KV head `head`
  const float* vsrc = qkv + (size_t)r * (qd + 2 * kd) + qd + kd + head * hd;
  float v1 = vsrc[lane], v2 = vsrc[lane + half];
  const int b = ri.b;
  if (ri.is_mask) {
    int i = ri.t - P.A;   // block index
    size_t kb = (((size_t)b * hkv + head) * kpad + i) * hd;
    size_t vb = ((size_t)b * hkv + head) * hd * kpad;
    int col = vt_col(i);
    if (bf16) {
      ((uint16_t*)ks)[kb + lane] = f2bf(o1);
      ((uint16_t*)ks)[kb + lane + half] = f2bf(o2);
      ((uint16_t*)vs)[vb + (size_t)lane * kpad + col] = f2bf(v1);
      ((uint16_t*)vs)[vb + (size_t)(lane + half) * kpad + col] = f2bf(v2);
    } else {
      ((float*)ks)[kb + lane] = o1;
      ((float*)ks)[kb + lane + half] = o2;
      ((float*)vs)[vb + (size_t)lane * kpad + col] = v1;
      ((float*)vs)[vb + (size_t)(lane + half) * kpad + col] = v2;
    }
  } else {
    const int p = ri.pos;
    if (p >= cap) return;       // the host bound makes this unreachable
    size_t kb = (((size_t)b * hkv + head) * cap + p) * hd;
    size_t vb = (((size_t)b * hkv + head) * (cap / 64) + p / 64) * (size_t)hd * 64;
    int col = vt_col(p & 63);
    if (bf16) {
      ((uint16_t*)kc)[kb + lane] = f2bf(o1);
      ((uint16_t*)kc)[kb + lane + half] = f2bf(o2);
      ((uint16_t*)vc)[vb + (size_t)lane * 64 + col] = f2bf(v1);
      ((uint16_t*)vc)[vb + (size_t)(lane + half) * 64 + col] = f2bf(v2);
    } else {
      ((float*)kc)[kb + lane] = o1;
      ((float*)kc)[kb + lane + half] = o2;
      ((float*)vc)[vb + (size_t)lane * 64 + col] = v1;
      ((float*)vc)[vb + (size_t)(lane + half) * 64 + col] = v2;
    }
  }
}

void launch_qkv_post(const PassInfo& P, const float* qkv, int hq, int hkv, int hd,
                     const void* qn, const void* kn, const void* dqn, const void* dkn, bool bf16,
                     float eps, const float* rope, void* q_out, void* kc, void* vc, int cap,
                     void* ks, void* vs, int kpad, hipStream_t s) {
  int rows = P.rows();
  if (rows <= 0) return;
  hipLaunchKernelGGL(k_qkv_post, dim3(rows, hq + hkv), dim3(64), 0, s, P, qkv, hq, hkv, hd, qn,
                     kn, dqn, dkn, (int)bf16, eps, (const float2*)rope, q_out, kc, vc, cap, ks, vs,
                     kpad);
}

// ---------------------------------------------------- LM-head argmax
// Partials are (value, index) per (row, column range), ranges ascending; a
// later range wins only if strictly larger, so ties go to the lowest index.
__global__ void k_lm_reduce(const float2* __restrict__ part, int rows, int nparts, PassInfo P,
                            int K, int32_t* __restrict__ drafts, int32_t* __restrict__ ar,
                            int32_t* __restrict__ pending) {
  int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const float2* p = part + (size_t)r * nparts;
  float best = p[0].x;
  int idx = __float_as_int(p[0].y);
  for (int j = 1; j < nparts; ++j) {
    float v = p[j].x;
    if (v > best) { best = v; idx = __float_as_int(p[j].y); }
  }
  const RowInfo ri = row_info(P, r);
  if (ri.pad) return;
  if (P.kind == PASS_DRAFT) {
    if (!ri.is_mask) {
      if (pending) pending[ri.b] = idx; else ar[(size_t)ri.b * (K + 1)] = idx;
    } else {
      drafts[(size_t)ri.b * K + (ri.t - P.A)] = idx;
    }
  } else if (P.kind == PASS_VERIFY) {
    ar[(size_t)ri.b * (K + 1) + 1 + ri.t] = idx;
  }
}

void launch_lm_reduce(const float2* part, int rows, int nparts, const PassInfo& P, int K,
                      int32_t* drafts, int32_t* ar_tokens, int32_t* pending, hipStream_t s) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(k_lm_reduce, dim3((rows + 63) / 64), dim3(64), 0, s, part, rows, nparts, P,
                     K, drafts, ar_tokens, pending);
}

// ------------------------------------------------------------ accept
// One wave per sequence: lane i compares d_{i+1} with a_i; the accept length
// is the index of the lowest lane that disagrees (K if none).
__global__ __launch_bounds__(64) void k_accept(int K, int ld, const int32_t* __restrict__ drafts,
                                               const int32_t* __restrict__ ar,
                                               int32_t* __restrict__ accept_len) {
  int b = blockIdx.x, lane = threadIdx.x;
  bool ne = false;
  if (lane < K) ne = drafts[(size_t)b * ld + lane] != ar[(size_t)b * (ld + 1) + lane];
  unsigned long long mask = __ballot(ne);
  if (lane == 0) accept_len[b] = mask ? (int)__ffsll((long long)mask) - 1 : K;
}

void launch_accept(int B, int K, int ld, const int32_t* drafts, const int32_t* ar,
                   int32_t* accept_len, hipStream_t s) {
  hipLaunchKernelGGL(k_accept, dim3(B), dim3(64), 0, s, K, ld, drafts, ar, accept_len);
}

// ------------------------------------------------------------ commit
// One 256-thread block; thread b handles sequence b.  Output offsets are an
// exclusive prefix sum of (m_b + 1): a wave scan plus a scan of wave totals.
__global__ __launch_bounds__(256) void k_commit(int B, int ld, const int32_t* __restrict__ acc,
                                                const int32_t* __restrict__ ar,
                                                const int32_t* __restrict__ drafts,
                                                int32_t* __restrict__ seq_len,
                                                int32_t* __restrict__ pending,
                                                int32_t* __restrict__ commit_start,
                                                int32_t* __restrict__ out_tokens,
                                                int32_t* __restrict__ out_off) {
  __shared__ int wsum[4];
  int b = threadIdx.x, lane = b & 63, w = b >> 6;
  int m = 0, cnt = 0;
  if (b < B) { m = acc[b]; cnt = m + 1; }
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0;
  for (int j = 0; j < w; ++j) base += wsum[j];
  int off = base + incl - cnt;
  if (b < B) {
    int n = seq_len[b];
    commit_start[b] = n;
    seq_len[b] = n + 1 + m;
    int bonus = ar[(size_t)b * (ld + 1) + m];
    pending[b] = bonus;
    for (int j = 0; j < m; ++j) out_tokens[off + j] = drafts[(size_t)b * ld + j];
    out_tokens[off + m] = bonus;
    out_off[b] = off;
    if (b == B - 1) out_off[B] = off + cnt;
  }
}

void launch_commit(int B, int ld, const int32_t* accept_len, const int32_t* ar,
                   const int32_t* drafts, int32_t* seq_len, int32_t* pending,
                   int32_t* commit_start, int32_t* out_tokens, int32_t* out_off, hipStream_t s) {
  hipLaunchKernelGGL(k_commit, dim3(1), dim3(256), 0, s, B, ld, accept_len, ar, drafts, seq_len,
                     pending, commit_start, out_tokens, out_off);
}

// ----------------------------------------------------- prefill helpers
__global__ void k_prefill_tail(int B, const int32_t* __restrict__ tokens, int ld,
                               const int32_t* __restrict__ plen, int pmax,
                               int32_t* __restrict__ seq_len, int32_t* __restrict__ last_tok) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int p = plen[b];
  p = p < 1 ? 1 : (p > pmax ? pmax : p);
  seq_len[b] = p - 1;
  last_tok[b] = tokens[(size_t)b * ld + p - 1];
}

void launch_prefill_tail(int B, const int32_t* tokens, int ld, const int32_t* plen_dev, int pmax,
                         int32_t* seq_len, int32_t* last_tok, hipStream_t s) {
  hipLaunchKernelGGL(k_prefill_tail, dim3((B + 63) / 64), dim3(64), 0, s, B, tokens, ld, plen_dev,
                     pmax, seq_len, last_tok);
}

__global__ void k_len_add(int B, int32_t* seq_len, int add) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) seq_len[b] += add;
}

void launch_len_add(int B, int32_t* seq_len, int add, hipStream_t s) {
  hipLaunchKernelGGL(k_len_add, dim3((B + 63) / 64), dim3(64), 0, s, B, seq_len, add);
}

// Read-bandwidth probe (measurement aid, not part of the decode step): every
// workgroup streams a contiguous share of the buffer with 16-byte loads, 8
// per lane in flight, and folds the words with XOR into one value per
// workgroup, so no load is dead.
__global__ __launch_bounds__(256) void k_stream_read(const u32x4_t* __restrict__ p, uint64_t n16,
                                                     uint32_t* __restrict__ out) {
  __shared__ uint32_t red[4];
  const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const uint64_t lo = (uint64_t)blockIdx.x * per;
  const uint64_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  for (uint64_t i = lo + threadIdx.x; i < hi; i += 256 * 8) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint64_t j = i + (uint64_t)u * 256;
      v[u] = j < hi ? __builtin_nontemporal_load(p + j) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

void launch_stream_read(const void* buf, uint64_t bytes, uint32_t* out, int nwg, hipStream_t s) {
  hipLaunchKernelGGL(k_stream_read, dim3(nwg), dim3(256), 0, s, (const u32x4_t*)buf, bytes / 16, out);
}

