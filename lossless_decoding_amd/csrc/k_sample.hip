// Sampling at temperature T > 0 with lossless rejection sampling.
//
// The pages state only that sampling with T > 0 relies on rejection
// sampling (HN item page, "Limitations"; atlas.scime.ai page,
// "Limitations").  The rule taken is the standard speculative-sampling one,
// in the step shape of this library: the anchor row's AR distribution p_0
// (pass 1) and the verify rows' p_1..p_K (pass 2) are softmax(z / T) of the
// frozen view's logits; the diffusion view's mask rows give q_1..q_K.
//   drafts      d_i ~ q_i, independently for every mask row;
//   acceptance  d_i is accepted with probability min(1, p_{i-1}(d_i) /
//               q_i(d_i)), in order, until the first rejection; m accepted;
//   final token on a rejection of d_{m+1}: a sample of the residual
//               max(0, p_m - q_{m+1}) renormalised; if all K are accepted:
//               a sample of p_K (the bonus).
// Every emitted token is then distributed as the AR model's own sample at
// its position, whatever q is.
//
// Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC'11), key = the context's seed,
// counter = (index, sequence, step, purpose); the first output word x0 is
// the uniform (x0 >> 8) * 2^-24 in [0, 1).  Purposes: 1 = drawing mask row
// i's draft (index i), 2 = accepting draft i (index i), 3 = the final token
// (index 0).
//
// Categorical sampling from weights w_j = 2^((z_j - M) * log2(e) / T)
// (M = the row maximum): 256 threads each own a contiguous chunk of the
// vocabulary, chunk sums are added in thread order, and the token is the
// first j whose running sum exceeds u * (sum of all w).  Every sum runs in a
// fixed order, so a row's result depends only on its own logits and u.
#include "internal.h"

namespace {

__device__ __forceinline__ uint32_t mulhi32(uint32_t a, uint32_t b) {
  return (uint32_t)(((uint64_t)a * b) >> 32);
}

// Philox4x32 with 10 rounds; returns the first output word.
__device__ __forceinline__ uint32_t philox_x0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                              uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = M0 * c0, hi0 = mulhi32(M0, c0);
    const uint32_t lo1 = M1 * c2, hi1 = mulhi32(M1, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += W0; k1 += W1;
  }
  return c0;
}

__device__ __forceinline__ float uniform01(const SampleArgs& s, int purpose, int index, int b) {
  const uint32_t x = philox_x0((uint32_t)index, (uint32_t)b, (uint32_t)s.step, (uint32_t)purpose,
                               (uint32_t)s.seed, (uint32_t)(s.seed >> 32));
  return (float)(x >> 8) * (1.0f / 16777216.0f);
}

constexpr int NT = 256;

// Block-wide reductions in a fixed tree (thread order).
__device__ __forceinline__ float block_max(float v, float* red) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int w = NT / 2; w > 0; w >>= 1) {
    if (t < w) red[t] = fmaxf(red[t], red[t + w]);
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

// Exclusive prefix of the per-thread values in thread order (one thread
// adds them sequentially: 256 adds), and the total.
__device__ __forceinline__ float block_prefix(float v, float* red, float& total) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  if (t == 0) {
    float acc = 0.f;
    for (int i = 0; i < NT; ++i) { const float x = red[i]; red[i] = acc; acc += x; }
    red[NT] = acc;
  }
  __syncthreads();
  const float p = red[t];
  total = red[NT];
  __syncthreads();
  return p;
}

struct Chunk { int lo, hi; };
__device__ __forceinline__ Chunk chunk_of(int V) {
  const int C = (V + NT - 1) / NT;
  Chunk c;
  c.lo = min(V, threadIdx.x * C);
  c.hi = min(V, c.lo + C);
  return c;
}

// The token of a chunk at which the running sum of its weights first
// exceeds t (relative to the chunk's start); the chunk's last token of
// nonzero weight if rounding leaves the sum at or below t.
template <typename Wt>
__device__ __forceinline__ int walk(const Chunk& ch, float t, Wt weight) {
  float acc = 0.f;
  int last = ch.lo;
  for (int j = ch.lo; j < ch.hi; ++j) {
    const float w = weight(j);
    if (w > 0.f) {
      last = j;
      acc += w;
      if (acc > t) return j;
    }
  }
  return last;
}

// Per row: M = max logit, the weights' chunk sums and S = their total; a
// mask row of a drafting pass also draws its draft with u (purpose 1).
__global__ __launch_bounds__(NT) void k_row_stats_sample(SampleArgs s, PassInfo P,
                                                         const float* __restrict__ logits, int ld,
                                                         float2* __restrict__ stats,
                                                         int32_t* __restrict__ drafts, int Kb) {
  __shared__ float red[NT + 1];
  const int r = blockIdx.x;
  const RowInfo ri = row_info(P, r);
  if (ri.pad) return;
  const float* z = logits + (size_t)r * ld;
  const Chunk ch = chunk_of(s.V);
  float m = -INFINITY;
  for (int j = ch.lo; j < ch.hi; ++j) m = fmaxf(m, z[j]);
  const float M = block_max(m, red);
  const float sc = 1.4426950408889634f / s.T;
  float cs = 0.f;
  for (int j = ch.lo; j < ch.hi; ++j) cs += exp2f((z[j] - M) * sc);
  float S;
  const float pre = block_prefix(cs, red, S);
  if (threadIdx.x == 0) stats[r] = make_float2(M, S);
  if (!(P.kind == PASS_DRAFT && ri.is_mask && drafts)) return;
  const int i = ri.t - P.A;
  const float target = uniform01(s, 1, i, ri.b) * S;
  // the thread whose chunk holds the target walks it; past the total (a u
  // of nearly 1 against the rounded sum) the last token of nonzero weight
  if (pre <= target && target < pre + cs && cs > 0.f) {
    drafts[(size_t)ri.b * Kb + i] =
        walk(ch, target - pre, [&](int j) { return exp2f((z[j] - M) * sc); });
  }
  __syncthreads();
  if (threadIdx.x == 0 && !(target < S)) {
    int tok = s.V - 1;
    while (tok > 0 && !(exp2f((z[tok] - M) * sc) > 0.f)) --tok;
    drafts[(size_t)ri.b * Kb + i] = tok;
  }
}

// Acceptance and the final token, one workgroup per sequence.
__global__ __launch_bounds__(NT) void k_spec_accept(SampleArgs s, int K, int ld_tok,
                                                    const int32_t* __restrict__ drafts,
                                                    int32_t* __restrict__ ar,
                                                    int32_t* __restrict__ accept_len) {
  __shared__ float red[NT + 1];
  __shared__ int sm;
  const int b = blockIdx.x;
  const float sc = 1.4426950408889634f / s.T;
  // AR row of position n+1+i (p_i): the anchor (draft pass) for i = 0, verify
  // row i-1 after; the mask row of draft i (q_i, 1-based)
  auto prow = [&](int i, const float*& z, float2& st) {
    if (i == 0) {
      const int r = s.RM + b;
      z = s.dlogits + (size_t)r * s.V; st = s.dstats[r];
    } else {
      const int r = b * K + (i - 1);
      z = s.vlogits + (size_t)r * s.V; st = s.vstats[r];
    }
  };
  auto qrow = [&](int i, const float*& z, float2& st) {
    const int r = b * K + (i - 1);
    z = s.dlogits + (size_t)r * s.V; st = s.dstats[r];
  };
  if (threadIdx.x == 0) {
    int m = 0;
    for (; m < K; ++m) {
      const int d = drafts[(size_t)b * ld_tok + m];
      if (d < 0 || d >= s.V) break;                 // not a token: never accepted
      const float* zp; float2 sp; prow(m, zp, sp);
      const float* zq; float2 sq; qrow(m + 1, zq, sq);
      const float p = exp2f((zp[d] - sp.x) * sc) / sp.y;
      const float q = exp2f((zq[d] - sq.x) * sc) / sq.y;
      const float u = uniform01(s, 2, m + 1, b);
      if (!(u * q < p)) break;                      // accepted with probability min(1, p / q)
    }
    sm = m;
  }
  __syncthreads();
  const int m = sm;
  // final token: residual max(0, p_m - q_{m+1}) after a rejection, p_K after
  // K acceptances
  const float* zp; float2 sp; prow(m, zp, sp);
  const float* zq = nullptr; float2 sq = make_float2(0.f, 1.f);
  if (m < K) qrow(m + 1, zq, sq);
  auto weight = [&](int j) -> float {
    const float p = exp2f((zp[j] - sp.x) * sc) / sp.y;
    if (!zq) return p;
    const float q = exp2f((zq[j] - sq.x) * sc) / sq.y;
    return fmaxf(p - q, 0.f);
  };
  const Chunk ch = chunk_of(s.V);
  float cs = 0.f;
  for (int j = ch.lo; j < ch.hi; ++j) cs += weight(j);
  float R;
  const float pre = block_prefix(cs, red, R);
  const float target = uniform01(s, 3, 0, b) * R;
  __shared__ int stok;
  if (threadIdx.x == 0) stok = -1;
  __syncthreads();
  if (pre <= target && target < pre + cs && cs > 0.f) stok = walk(ch, target - pre, weight);
  __syncthreads();
  if (threadIdx.x == 0) {
    int tok = stok;
    if (tok < 0) {
      // the target fell past the rounded total, or the residual vanished in
      // rounding (p_m equal to q_{m+1} to fp32): the last token of nonzero
      // weight, else p_m's most likely token
      tok = s.V - 1;
      while (tok > 0 && !(weight(tok) > 0.f)) --tok;
      if (!(weight(tok) > 0.f)) {
        float best = -INFINITY;
        for (int j = 0; j < s.V; ++j)
          if (zp[j] > best) { best = zp[j]; tok = j; }
      }
    }
    int32_t* a = ar + (size_t)b * (ld_tok + 1);
    for (int i = 0; i < m; ++i) a[i] = drafts[(size_t)b * ld_tok + i];
    a[m] = tok;
    accept_len[b] = m;
  }
}

// The first generated token after a prefill at T > 0: a sample of the last
// prompt row's distribution (the anchor row RM + b of the prefill's last
// pass), purpose 4.
__global__ __launch_bounds__(NT) void k_sample_first(SampleArgs s, int RM,
                                                     const float* __restrict__ logits,
                                                     const float2* __restrict__ stats,
                                                     int32_t* __restrict__ pending) {
  __shared__ float red[NT + 1];
  __shared__ int stok;
  const int b = blockIdx.x, r = RM + b;
  const float* z = logits + (size_t)r * s.V;
  const float2 st = stats[r];
  const float sc = 1.4426950408889634f / s.T;
  auto weight = [&](int j) { return exp2f((z[j] - st.x) * sc); };
  const Chunk ch = chunk_of(s.V);
  float cs = 0.f;
  for (int j = ch.lo; j < ch.hi; ++j) cs += weight(j);
  float S;
  const float pre = block_prefix(cs, red, S);
  const float target = uniform01(s, 4, 0, b) * S;
  if (threadIdx.x == 0) stok = -1;
  __syncthreads();
  if (pre <= target && target < pre + cs && cs > 0.f) stok = walk(ch, target - pre, weight);
  __syncthreads();
  if (threadIdx.x == 0) {
    int tok = stok;
    if (tok < 0) {
      tok = s.V - 1;
      while (tok > 0 && !(weight(tok) > 0.f)) --tok;
    }
    pending[b] = tok;
  }
}

}  // namespace

void launch_sample_first(const SampleArgs& s, int B, int RM, const float* logits,
                         const float2* stats, int32_t* pending, hipStream_t st) {
  hipLaunchKernelGGL(k_sample_first, dim3(B), dim3(NT), 0, st, s, RM, logits, stats, pending);
}

void launch_sample_rows(const SampleArgs& s, const PassInfo& P, const float* logits, int ld,
                        float2* stats, int32_t* drafts, int Kb, hipStream_t st) {
  const int rows = P.rows();
  if (rows <= 0) return;
  hipLaunchKernelGGL(k_row_stats_sample, dim3(rows), dim3(NT), 0, st, s, P, logits, ld, stats,
                     drafts, Kb);
}

void launch_spec_accept(const SampleArgs& s, int B, int K, int ld_tok, const int32_t* drafts,
                        int32_t* ar, int32_t* accept_len, hipStream_t st) {
  hipLaunchKernelGGL(k_spec_accept, dim3(B), dim3(NT), 0, st, s, K, ld_tok, drafts, ar,
                     accept_len);
}
