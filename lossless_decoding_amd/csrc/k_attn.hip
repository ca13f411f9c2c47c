// Block attention over the shared KV cache (the draft pass's anchor + mask
// rows, the verify pass's causal rows, prefill rows).
//
// bf16 path.  One workgroup per (sequence, KV head, key chunk).  All query
// rows of the pass for that sequence and every query head of the GQA group
// (T tokens x G heads, at most 144 rows = 9 row tiles of 16) share each
// 64-key K/V tile staged in LDS, so the cache is streamed once per pass.
// MFMA: S^T = K . Q^T (keys x rows) and O^T = V^T . P^T (dims x rows), so a
// lane always holds one query row and the softmax statistics stay in-lane.
// Online softmax in fp32 (base-2 exponent).  Chunks are SC keys aligned to
// absolute cache positions; each chunk's partial (max, sum, unnormalised
// output) is folded in increasing chunk order by the merge kernel, and the
// draft block's keys are folded last.  A row's result therefore depends only
// on which keys it sees, never on the other rows of the pass: fully masked
// tiles and chunks are exact no-ops, masked keys are removed by selection
// (never by multiplying stale values), and keys past the pass's last
// written slot are zeroed when staged.
//
// fp32 path: one wave per (row, query head), keys in order (check models).
#include "internal.h"

#define KT_STRIDE 136   // bf16 per key row of the staged K tile (128 + 8 pad)
#define VT_STRIDE 72    // bf16 per dimension row of the staged V^T tile (64 + 8 pad)
#define AT_MAX_RT_PER_WAVE 3

__device__ __forceinline__ bf16x8_t ld_bf16x8(const uint16_t* p) {
  uint4 v = *(const uint4*)p;
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// key index (0..63) stored at column c of a V^T tile (inverse of vt_col)
__device__ __forceinline__ int vt_key(int c) {
  int g = c >> 5, k = c & 31;
  int q = k >> 3, h = (k >> 2) & 1, i = k & 3;
  return g * 32 + h * 16 + q * 4 + i;
}

struct SeqLimits {
  int maxlim;     // last cache slot any row of this sequence may see
  int n;          // committed length (draft/verify)
};

__device__ __forceinline__ SeqLimits seq_limits(const AttnArgs& a, int b) {
  SeqLimits L;
  const PassInfo& P = a.P;
  if (a.fixed_ctx >= 0) { L.n = a.fixed_ctx; L.maxlim = a.fixed_ctx - 1; return L; }
  if (P.kind == PASS_DRAFT) { L.n = P.len[b]; L.maxlim = L.n; }
  else if (P.kind == PASS_VERIFY) { L.n = P.len[b]; L.maxlim = L.n + P.Kx; }
  else { L.n = 0; L.maxlim = P.p0 + P.Kx - 1; }
  return L;
}

// last visible cache slot of token t of sequence b (-1: none), and whether
// it sees the draft block
__device__ __forceinline__ void token_view(const AttnArgs& a, const SeqLimits& L, int t,
                                           int& limit, int& sees_block) {
  const PassInfo& P = a.P;
  if (a.fixed_ctx >= 0) { limit = a.fixed_ctx - 1; sees_block = 1; return; }
  if (P.kind == PASS_DRAFT) { limit = L.n; sees_block = t >= P.A; return; }
  sees_block = 0;
  limit = P.kind == PASS_VERIFY ? L.n + 1 + t : P.p0 + t;
}

__global__ __launch_bounds__(256) void k_attn_bf16(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[64 * KT_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[128 * VT_STRIDE];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
  const PassInfo& P = a.P;
  const int T = a.fixed_ctx >= 0 ? P.Kx : P.tokens_per_seq();
  const int G = a.hq / a.hkv;
  const int QR = T * G;
  const int NRT = (QR + 15) >> 4;
  const bool blk = (c == a.nc);
  const int hd = 128;
  const int H = a.hq * hd;

  if (blk && !(a.block_len > 0 && (a.fixed_ctx >= 0 || (P.kind == PASS_DRAFT && P.Kx > 0))))
    return;
  const SeqLimits L = seq_limits(a, b);
  int k_begin, k_end;
  if (!blk) {
    k_begin = c * a.sc;
    if (k_begin > L.maxlim) return;
    k_end = min(min(k_begin + a.sc, L.maxlim + 1), a.cap);
  } else {
    k_begin = 0;
    k_end = a.block_len;
  }

  // query fragments (B operand of S^T = K.Q^T): row qr = rt*16 + lr
  bf16x8_t qf[AT_MAX_RT_PER_WAVE][4];
  int lim[AT_MAX_RT_PER_WAVE], seesb[AT_MAX_RT_PER_WAVE];
  floatx4_t oacc[AT_MAX_RT_PER_WAVE][8];
  float mrow[AT_MAX_RT_PER_WAVE], lrow[AT_MAX_RT_PER_WAVE];
#pragma unroll
  for (int j = 0; j < AT_MAX_RT_PER_WAVE; ++j) {
    int rt = wave + 4 * j;
    int qr = rt * 16 + lr;
    lim[j] = -1; seesb[j] = 0;
    mrow[j] = -INFINITY; lrow[j] = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[j][db] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    if (rt < NRT && qr < QR) {
      int t = qr / G, hh = g * G + (qr - t * G);
      int r = row_of(P, b, t);
      token_view(a, L, t, lim[j], seesb[j]);
      const uint16_t* qp = (const uint16_t*)a.q + (size_t)r * H + hh * hd + lq * 8;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) qf[j][ds] = ld_bf16x8(qp + ds * 32);
    } else {
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) qf[j][ds] = bf16x8_t{};
    }
  }

  const uint16_t* kbase;
  const uint16_t* vbase;
  if (!blk) {
    kbase = (const uint16_t*)a.kc + ((size_t)b * a.hkv + g) * a.cap * hd;
    vbase = (const uint16_t*)a.vc + ((size_t)b * a.hkv + g) * a.cap * hd;   // tiles of 64*hd
  } else {
    kbase = (const uint16_t*)a.ks + ((size_t)b * a.hkv + g) * a.kpad * hd;
    vbase = (const uint16_t*)a.vs + ((size_t)b * a.hkv + g) * hd * a.kpad;
  }
  const float sl2 = 1.4426950408889634f / sqrtf((float)hd);

  for (int kt = k_begin; kt < k_end; kt += 64) {
    const int nvalid = min(64, k_end - kt);
    // ---- stage K (64 x 128) and V^T (128 x 64) into LDS, zeroing keys >= nvalid
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int ci = tid + j * 256;
      int key = ci >> 4, col = (ci & 15) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (key < nvalid) v = *(const uint4*)(kbase + (size_t)(kt + key) * hd + col);
      *(uint4*)(sK + key * KT_STRIDE + col) = v;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int ci = tid + j * 256;
      int d = ci >> 3, col = (ci & 7) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (!blk) {
        v = *(const uint4*)(vbase + (size_t)(kt >> 6) * 64 * hd + (size_t)d * 64 + col);
      } else if (col < a.kpad) {
        v = *(const uint4*)(vbase + (size_t)d * a.kpad + col);
      }
      if (nvalid < 64) {
        uint16_t e[8];
        __builtin_memcpy(e, &v, 16);
#pragma unroll
        for (int x = 0; x < 8; ++x)
          if (vt_key(col + x) >= nvalid) e[x] = 0;
        __builtin_memcpy(&v, e, 16);
      }
      *(uint4*)(sV + d * VT_STRIDE + col) = v;
    }
    __syncthreads();

#pragma unroll
    for (int j = 0; j < AT_MAX_RT_PER_WAVE; ++j) {
      int rt = wave + 4 * j;
      if (rt >= NRT) continue;
      // S^T for 4 blocks of 16 keys
      floatx4_t s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) {
          bf16x8_t kf = ld_bf16x8(sK + (kb * 16 + lr) * KT_STRIDE + ds * 32 + lq * 8);
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[j][ds], s[kb], 0, 0, 0);
        }
      }
      // mask by selection and scale to base 2
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int kl = kb * 16 + lq * 4 + i;
          bool ok = kl < nvalid && (blk ? seesb[j] != 0 : (kt + kl) <= lim[j]);
          float v = ok ? s[kb][i] * sl2 : -INFINITY;
          s[kb][i] = v;
          mt = fmaxf(mt, v);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      // Branch-free update: the MFMAs below read operands from every lane,
      // so no lane may skip them.  A row with nothing visible yet keeps
      // m = -inf, l = 0, o = 0 exactly (alpha = 1, p = 0).
      const float mnew = fmaxf(mrow[j], mt);
      const bool any = mnew != -INFINITY;
      const float mref = any ? mnew : 0.f;
      const float alpha = any ? exp2f(mrow[j] - mref) : 1.f;
      // P enters the P.V product as two bf16 terms, hi = bf16(p) and
      // lo = bf16(p - hi) (p - hi is exact in fp32), so the product carries
      // about 16 significant bits of p instead of 8.  Rounding p itself to
      // bf16 would make the result depend on the running maximum it was
      // taken against, i.e. on how the keys were split into tiles and chunks.
      float ps = 0.f;
      bf16x8_t pf[2], pl[2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p = exp2f(s[kb][i] - mref);
          ps += p;
          __bf16 hi = (__bf16)p;
          pf[kb >> 1][(kb & 1) * 4 + i] = hi;
          pl[kb >> 1][(kb & 1) * 4 + i] = (__bf16)(p - (float)hi);
        }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      lrow[j] = lrow[j] * alpha + ps;
      mrow[j] = any ? mnew : mrow[j];
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        floatx4_t o = oacc[j][db];
        o[0] *= alpha; o[1] *= alpha; o[2] *= alpha; o[3] *= alpha;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8_t vf = ld_bf16x8(sV + (db * 16 + lr) * VT_STRIDE + ks * 32 + lq * 8);
          o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[ks], o, 0, 0, 0);
          o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl[ks], o, 0, 0, 0);
        }
        oacc[j][db] = o;
      }
    }
    __syncthreads();
  }

  // partials: opart[((b*hkv+g)*(nc+1)+c)*qr_max + qr][d], ml[...][2]
  const size_t pbase = ((size_t)(b * a.hkv + g) * (a.nc + 1) + c) * a.qr_max;
#pragma unroll
  for (int j = 0; j < AT_MAX_RT_PER_WAVE; ++j) {
    int rt = wave + 4 * j;
    int qr = rt * 16 + lr;
    if (rt >= NRT || qr >= QR) continue;
    float* op = a.opart + (pbase + qr) * hd;
#pragma unroll
    for (int db = 0; db < 8; ++db) *(floatx4_t*)(op + db * 16 + lq * 4) = oacc[j][db];
    if (lq == 0) {
      a.ml[(pbase + qr) * 2 + 0] = mrow[j];
      a.ml[(pbase + qr) * 2 + 1] = lrow[j];
    }
  }
}

// Fold the chunk partials of one (row, query head) in increasing chunk
// order, then the block chunk for rows that see the draft block.
__global__ __launch_bounds__(64) void k_attn_merge(AttnArgs a) {
  const int r = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const PassInfo& P = a.P;
  const int hd = a.hd, G = a.hq / a.hkv, g = h / G;
  int b, t;
  if (a.fixed_ctx >= 0) { b = r / P.Kx; t = r - b * P.Kx; }
  else {
    RowInfo ri = row_info(P, r);
    if (ri.pad) return;
    b = ri.b; t = ri.t;
  }
  const SeqLimits L = seq_limits(a, b);
  int limit, sees;
  token_view(a, L, t, limit, sees);
  const int qr = t * G + (h - g * G);
  if (limit >= a.cap) limit = a.cap - 1;
  const int nchunks = limit >= 0 ? limit / a.sc + 1 : 0;
  float m = -INFINITY, l = 0.f;
  float o0 = 0.f, o1 = 0.f;
  const size_t sbase = (size_t)(b * a.hkv + g) * (a.nc + 1);
  for (int c = 0; c <= nchunks; ++c) {
    int cc = c;
    if (c == nchunks) {
      if (!(sees && a.block_len > 0)) break;
      cc = a.nc;
    }
    size_t pi = (sbase + cc) * a.qr_max + qr;
    float mc = a.ml[pi * 2], lc = a.ml[pi * 2 + 1];
    if (mc == -INFINITY) continue;
    float mn = fmaxf(m, mc);
    float al = exp2f(m - mn), be = exp2f(mc - mn);
    const float* op = a.opart + pi * hd;
    l = l * al + lc * be;
    o0 = o0 * al + op[lane * 2] * be;
    o1 = o1 * al + op[lane * 2 + 1] * be;
    m = mn;
  }
  float inv = 1.0f / l;
  size_t ob = (size_t)r * a.hq * hd + (size_t)h * hd + lane * 2;
  uint16_t y0 = f2bf(o0 * inv), y1 = f2bf(o1 * inv);
  ((uint16_t*)a.out)[ob] = y0;
  ((uint16_t*)a.out)[ob + 1] = y1;
  if (a.tap && r < a.tap_rows) {
    ((uint16_t*)a.tap)[ob] = y0;
    ((uint16_t*)a.tap)[ob + 1] = y1;
  }
}

void launch_attention_bf16(const AttnArgs& a, hipStream_t s) {
  const int B = a.P.B;
  hipLaunchKernelGGL(k_attn_bf16, dim3(a.nc + 1, a.hkv, B), dim3(256), 0, s, a);
  int rows = a.fixed_ctx >= 0 ? B * a.P.Kx : a.P.rows();
  hipLaunchKernelGGL(k_attn_merge, dim3(rows, a.hq), dim3(64), 0, s, a);
}

// ------------------------------------------------------------- fp32
__global__ __launch_bounds__(64) void k_attn_f32(AttnArgs a) {
  const int r = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const PassInfo& P = a.P;
  const int hd = a.hd, G = a.hq / a.hkv, g = h / G;
  RowInfo ri = row_info(P, r);
  if (ri.pad) return;
  const SeqLimits L = seq_limits(a, ri.b);
  int limit, sees;
  token_view(a, L, ri.t, limit, sees);
  const float* q = (const float*)a.q + (size_t)r * a.hq * hd + (size_t)h * hd;
  const float q0 = lane < hd ? q[lane] : 0.f;
  const float q1 = lane + 64 < hd ? q[lane + 64] : 0.f;
  const float scale = 1.0f / sqrtf((float)hd);
  const float* kc = (const float*)a.kc + ((size_t)ri.b * a.hkv + g) * a.cap * hd;
  const float* vc = (const float*)a.vc + ((size_t)ri.b * a.hkv + g) * a.cap * hd;
  const float* ks = (const float*)a.ks + ((size_t)ri.b * a.hkv + g) * a.kpad * hd;
  const float* vs = (const float*)a.vs + ((size_t)ri.b * a.hkv + g) * hd * a.kpad;
  const int nblk = (sees && P.kind == PASS_DRAFT) ? P.Kx : 0;
  if (limit >= a.cap) limit = a.cap - 1;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int j = 0; j <= limit + nblk; ++j) {
    const float* kr;
    float v0, v1;
    if (j <= limit) {
      kr = kc + (size_t)j * hd;
      const float* vt = vc + (size_t)(j >> 6) * 64 * hd;
      int col = vt_col(j & 63);
      v0 = lane < hd ? vt[(size_t)lane * 64 + col] : 0.f;
      v1 = lane + 64 < hd ? vt[(size_t)(lane + 64) * 64 + col] : 0.f;
    } else {
      int i = j - limit - 1;
      kr = ks + (size_t)i * hd;
      int col = vt_col(i);
      v0 = lane < hd ? vs[(size_t)lane * a.kpad + col] : 0.f;
      v1 = lane + 64 < hd ? vs[(size_t)(lane + 64) * a.kpad + col] : 0.f;
    }
    float part = q0 * (lane < hd ? kr[lane] : 0.f) + q1 * (lane + 64 < hd ? kr[lane + 64] : 0.f);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    float sc = part * scale;
    float mn = fmaxf(m, sc);
    float al = expf(m - mn), p = expf(sc - mn);
    l = l * al + p;
    o0 = o0 * al + p * v0;
    o1 = o1 * al + p * v1;
    m = mn;
  }
  float inv = 1.0f / l;
  float* out = (float*)a.out + (size_t)r * a.hq * hd + (size_t)h * hd;
  if (lane < hd) out[lane] = o0 * inv;
  if (lane + 64 < hd) out[lane + 64] = o1 * inv;
  if (a.tap && r < a.tap_rows) {
    float* tp = (float*)a.tap + (size_t)r * a.hq * hd + (size_t)h * hd;
    if (lane < hd) tp[lane] = o0 * inv;
    if (lane + 64 < hd) tp[lane + 64] = o1 * inv;
  }
}

void launch_attention_f32(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_attn_f32, dim3(a.P.rows(), a.hq), dim3(64), 0, s, a);
}
