// Block attention over the shared KV cache (the draft pass's anchor + mask
// rows, the verify pass's causal rows, prefill rows).
//
// bf16 path.  A workgroup handles (key chunk, KV head, sequence,
// group of four 16-row query tiles); the query rows of a sequence are its
// tokens x the G query heads of the KV head, so each 64-key K/V tile staged
// in LDS serves the whole GQA group.  A wave owns one query tile.
// MFMA: S^T = K . Q^T (keys x rows) and O^T = V^T . P^T (dims x rows), so a
// lane always holds one query row and the softmax statistics stay in-lane.
// Online softmax in fp32 (base-2 exponent); the next K/V tile is loaded into
// registers while the current one is computed.  Chunks are SC keys aligned
// to absolute cache positions; each writes its partial (max, sum,
// unnormalised output) and the merge kernel combines a row's partials in
// increasing chunk order, the draft block's keys last.  A row's result
// therefore depends only on which keys it sees, never on the other rows of
// the pass: fully masked tiles and chunks are exact no-ops, masked keys are
// removed by selection (never by multiplying stale values), and keys past
// the pass's last written slot are zeroed when staged.
//
// fp32 path: one wave per (row, query head), keys in order (check models).
#include "internal.h"

#define KT_STRIDE 136   // bf16 per key row of the staged K tile (128 + 8 pad)
#define VT_STRIDE 72    // bf16 per dimension row of the staged V^T tile (64 + 8 pad)

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

// number of 4-tile query row groups of a pass
__host__ __device__ inline int attn_row_groups(int qr) { return ((qr + 15) / 16 + 3) / 4; }

__global__ __launch_bounds__(256, 2) void k_attn_bf16(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[64 * KT_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[128 * VT_STRIDE];
  const int c = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
  const PassInfo& P = a.P;
  const int T = a.fixed_ctx >= 0 ? P.Kx : P.tokens_per_seq();
  const int G = a.hq / a.hkv;
  const int QR = T * G;
  const int NRT = (QR + 15) >> 4;
  const int NRG = attn_row_groups(QR);
  const int b = blockIdx.z / NRG, rg = blockIdx.z - b * NRG;
  const bool blk = (c == a.nc);
  const int hd = 128;
  const int H = a.hq * hd;

  // which chunks take part: every chunk up to the sequence's last visible
  // slot, plus the block chunk when the pass has a draft block
  const bool has_blk = a.block_len > 0 && (a.fixed_ctx >= 0 || (P.kind == PASS_DRAFT && P.Kx > 0));
  const SeqLimits L = seq_limits(a, b);
  const int lastk = L.maxlim < a.cap - 1 ? L.maxlim : a.cap - 1;
  const int nch = lastk >= 0 ? lastk / a.sc + 1 : 0;
  if (blk ? !has_blk : c >= nch) return;
  int k_begin, k_end;
  if (!blk) {
    k_begin = c * a.sc;
    k_end = min(k_begin + a.sc, lastk + 1);
  } else {
    k_begin = 0;
    k_end = a.block_len;
  }

  // this wave's query tile: row qr = rt*16 + lr (B operand of S^T = K.Q^T)
  const int rt = rg * 4 + wave;
  const int qr = rt * 16 + lr;
  const bool wact = rt < NRT;                 // uniform per wave
  bf16x8_t qf[4];
  int lim = -1, seesb = 0;
  floatx4_t oacc[8];
  float mrow = -INFINITY, lrow = 0.f;
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  if (wact && qr < QR) {
    const int t = qr / G, hh = g * G + (qr - t * G);
    const int r = row_of(P, b, t);
    token_view(a, L, t, lim, seesb);
    const uint16_t* qp = (const uint16_t*)a.q + (size_t)r * H + hh * hd + lq * 8;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) qf[ds] = ld_bf16x8(qp + ds * 32);
  } else {
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) qf[ds] = bf16x8_t{};
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

  // K (64 x 128) and V^T (128 x 64) of one tile: 4 + 4 16-byte pieces per
  // thread.  Two register sets alternate, so the tile two steps ahead is in
  // flight while one is computed.  The loads are buffer loads whose
  // descriptors end at this chunk's last key (K: whole keys; V: whole 64-key
  // tiles, the partial last tile is zeroed when staged): loads past the end
  // return zero without touching memory, so every load is issued
  // unconditionally and the memory-counter waits never drain the other set.
  const int kv_hi = blk ? a.block_len : k_end;                 // keys [0, kv_hi) exist
  const __amdgpu_buffer_rsrc_t rK =
      __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, kv_hi * hd * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc(
      (void*)vbase, (short)0, blk ? hd * a.kpad * 2 : ((kv_hi + 63) >> 6) * 64 * hd * 2, 0x00020000);
  uint4 kA[4], vA[4], kB[4], vB[4];
  auto load_tile = [&](uint4 (&kr)[4], uint4 (&vr)[4], int kt) __attribute__((always_inline)) {
    const bool live = kt < k_end;                              // uniform
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ci = tid + j * 256;
      const int key = ci >> 4, col = (ci & 15) * 8;
      const int ko = live ? ((kt + key) * hd + col) * 2 : 0x40000000;
      kr[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rK, ko, 0, 0));
      const int d = ci >> 3, vc8 = (ci & 7) * 8;
      const int vo = !live ? 0x40000000
                           : (blk ? (d * a.kpad + vc8) * 2 : ((kt >> 6) * 64 * hd + d * 64 + vc8) * 2);
      vr[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rV, vo, 0, 0));
    }
  };
  auto store_tile = [&](const uint4 (&kr)[4], const uint4 (&vr)[4], int kt) __attribute__((always_inline)) {
    const int nvalid = min(64, k_end - kt);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ci = tid + j * 256;
      const int key = ci >> 4, col = (ci & 15) * 8;
      *(uint4*)(sK + key * KT_STRIDE + col) = kr[j];
      const int d = ci >> 3, vc8 = (ci & 7) * 8;
      uint4 v = vr[j];
      if (nvalid < 64) {                 // zero the columns of keys past the end
        uint16_t e[8];
        __builtin_memcpy(e, &v, 16);
#pragma unroll
        for (int x = 0; x < 8; ++x)
          if (vt_key(vc8 + x) >= nvalid) e[x] = 0;
        __builtin_memcpy(&v, e, 16);
      }
      *(uint4*)(sV + d * VT_STRIDE + vc8) = v;
    }
  };

  // One tile step: stage the tile, refill its register set two tiles ahead,
  // compute.  A step past the end (odd tile count) sees no key: every score
  // is masked, alpha = 1 and p = 0, so it changes nothing.
  auto step = [&](uint4 (&kr)[4], uint4 (&vr)[4], int kt) __attribute__((always_inline)) {
    const int nvalid = min(64, k_end - kt);
    __syncthreads();                     // the previous tile is no longer read
    store_tile(kr, vr, kt);
    __syncthreads();
    load_tile(kr, vr, kt + 128);
    if (wact) {
      // S^T for 4 blocks of 16 keys
      floatx4_t s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) {
          bf16x8_t kf = ld_bf16x8(sK + (kb * 16 + lr) * KT_STRIDE + ds * 32 + lq * 8);
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ds], s[kb], 0, 0, 0);
        }
      }
      // Visibility: when every key of the tile is visible to every row of
      // the wave (the common case at long context) nothing is masked;
      // otherwise invisible keys get the score -inf.  Both paths then compute
      // the same values: the maximum of the raw scores, scaled to base 2
      // (scaling by a positive constant keeps the maximum), and
      // p = 2^(s * scale - m) with one fused multiply-add.
      const bool all_vis = !blk && nvalid == 64 && __all(kt + 63 <= lim);
      if (!all_vis) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kl = kb * 16 + lq * 4 + i;
            const bool ok = kl < nvalid && (blk ? seesb != 0 : (kt + kl) <= lim);
            s[kb][i] = ok ? s[kb][i] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mt = mx * sl2;
      // Branch-free update: the MFMAs below read operands from every lane,
      // so no lane may skip them.  A row with nothing visible yet keeps
      // m = -inf, l = 0, o = 0 exactly (alpha = 1, p = 0).
      const float mnew = fmaxf(mrow, mt);
      const bool any = mnew != -INFINITY;
      const float mref = any ? mnew : 0.f;
      const float alpha = any ? __builtin_amdgcn_exp2f(mrow - mref) : 1.f;
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
          // v_exp_f32 directly: the argument is <= 0 and results below
          // 2^-126 (flushed) are negligible softmax weights
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], sl2, -mref));
          ps += p;
          __bf16 hi = (__bf16)p;
          pf[kb >> 1][(kb & 1) * 4 + i] = hi;
          pl[kb >> 1][(kb & 1) * 4 + i] = (__bf16)(p - (float)hi);
        }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      lrow = lrow * alpha + ps;
      // rescale only if some row's maximum grew (otherwise every alpha is 1)
      if (__any(mnew != mrow)) {
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          oacc[db][0] *= alpha; oacc[db][1] *= alpha; oacc[db][2] *= alpha; oacc[db][3] *= alpha;
        }
      }
      mrow = any ? mnew : mrow;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        floatx4_t o = oacc[db];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8_t vf = ld_bf16x8(sV + (db * 16 + lr) * VT_STRIDE + ks * 32 + lq * 8);
          o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[ks], o, 0, 0, 0);
          o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl[ks], o, 0, 0, 0);
        }
        oacc[db] = o;
      }
    }
  };
  load_tile(kA, vA, k_begin);
  load_tile(kB, vB, k_begin + 64);
  for (int kt = k_begin; kt < k_end; kt += 128) {
    step(kA, vA, kt);
    step(kB, vB, kt + 64);
  }

  // ---- partial of this chunk: opart[((b*hkv+g)*(nc+1)+c)*qr_max + qr][d],
  // ml[...][2]
  if (wact && qr < QR) {
    const size_t pi = ((size_t)(b * a.hkv + g) * (a.nc + 1) + c) * a.qr_max + qr;
    float* op = a.opart + pi * hd;
#pragma unroll
    for (int db = 0; db < 8; ++db) *(floatx4_t*)(op + db * 16 + lq * 4) = oacc[db];
    if (lq == 0) {
      a.ml[pi * 2 + 0] = mrow;
      a.ml[pi * 2 + 1] = lrow;
    }
  }
}

// Combine the chunk partials of one (row, query head); one wave each, four
// per block.  Phase 1: the maximum M of the chunk maxima the row sees (its
// cache chunks, then the block chunk).  Phase 2: l = sum_c l_c 2^(m_c - M)
// and o = sum_c o_c 2^(m_c - M), summed in increasing chunk order (block
// last).  All loads of a phase are independent, so the merge costs two
// memory round trips; the result depends only on the row's own partials.
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a, int npairs) {
  __shared__ float sw[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + wave;
  if (pair >= npairs) return;
  const int r = pair / a.hq, h = pair - r * a.hq;
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
  const bool has_blk = a.block_len > 0 && (a.fixed_ctx >= 0 || (P.kind == PASS_DRAFT && P.Kx > 0));
  const int qr = t * G + (h - g * G);
  if (limit >= a.cap) limit = a.cap - 1;
  const int nrow = limit >= 0 ? limit / a.sc + 1 : 0;
  const int ntot = nrow + ((sees && has_blk) ? 1 : 0);   // partials this row folds
  const size_t sbase = (size_t)(b * a.hkv + g) * (a.nc + 1);
  auto pidx = [&](int j) { return (sbase + (j < nrow ? j : a.nc)) * a.qr_max + qr; };
  // phase 1: maxima (64 partials per pass over the lanes)
  float M = -INFINITY;
  for (int j0 = 0; j0 < ntot; j0 += 64) {
    const int j = j0 + lane;
    const float mc = j < ntot ? a.ml[pidx(j) * 2] : -INFINITY;
    M = fmaxf(M, mc);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  // phase 2: weights 2^(m_c - M) (0 for fully masked partials), then sums
  float l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int j0 = 0; j0 < ntot; j0 += 64) {
    const int j = j0 + lane;
    float wgt = 0.f, lw = 0.f;
    if (j < ntot) {
      const size_t pi = pidx(j);
      const float mc = a.ml[pi * 2], lc = a.ml[pi * 2 + 1];
      wgt = mc == -INFINITY ? 0.f : exp2f(mc - M);
      lw = lc * wgt;
    }
    sw[wave][lane] = wgt;
    // l in chunk order: gather the 64 products on every lane, add in order
    const int n = min(64, ntot - j0);
    float lws[1];
    lws[0] = lw;
    for (int k = 0; k < n; ++k) l += __shfl(lws[0], k, 64);
    __builtin_amdgcn_wave_barrier();
    // o: lane owns dimensions 2 lane, 2 lane + 1; loads in batches of 8
    for (int k0 = 0; k0 < n; k0 += 8) {
      float2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = k0 + u < n ? *(const float2*)(a.opart + pidx(j0 + k0 + u) * hd + lane * 2)
                          : make_float2(0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (k0 + u < n) {
          const float wu = sw[wave][k0 + u];
          o0 += v[u].x * wu;
          o1 += v[u].y * wu;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  const float inv = 1.0f / l;
  const size_t ob = (size_t)r * a.hq * hd + (size_t)h * hd + lane * 2;
  const uint32_t y = (uint32_t)f2bf(o0 * inv) | ((uint32_t)f2bf(o1 * inv) << 16);
  *(uint32_t*)((uint16_t*)a.out + ob) = y;
  if (a.tap && r < a.tap_rows) *(uint32_t*)((uint16_t*)a.tap + ob) = y;
}

void launch_attention_bf16(const AttnArgs& a, hipStream_t s) {
  const int B = a.P.B;
  const int T = a.fixed_ctx >= 0 ? a.P.Kx : a.P.tokens_per_seq();
  const int nrg = attn_row_groups(T * (a.hq / a.hkv));
  hipLaunchKernelGGL(k_attn_bf16, dim3(a.nc + 1, a.hkv, B * nrg), dim3(256), 0, s, a);
  const int rows = a.fixed_ctx >= 0 ? B * a.P.Kx : a.P.rows();
  const int npairs = rows * a.hq;
  hipLaunchKernelGGL(k_attn_merge, dim3((npairs + 3) / 4), dim3(256), 0, s, a, npairs);
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
