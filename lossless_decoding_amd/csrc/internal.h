// Internal declarations of liborthrus: pass descriptors, kernel launchers and
// the device helpers shared by the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "orthrus.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- passes
// Physical row order inside a pass.  Draft pass: the B*Kx mask rows first
// (row b*Kx + i), padding up to RM = a multiple of 16, then the A*B anchor
// rows (row RM + b).  Verify and prefill passes: B*Kx rows (row b*Kx + i).
// Putting the mask rows first makes both GEMM row groups start on a 16-row
// MFMA tile.
enum PassKind { PASS_DRAFT = 0, PASS_VERIFY = 1, PASS_PREFILL = 2 };

struct PassInfo {
  int kind;
  int B;             // sequences
  int A;             // 1 if anchor rows are present (draft passes)
  int Kx;            // block rows per sequence (masks / verified drafts / prompt rows)
  int p0;            // prefill: absolute position of block row 0
  int RM;            // draft: first anchor row (B*Kx rounded up to 16)
  const int32_t* len;  // device seq_len[B] (draft / verify)
  int refine;        // draft pass without anchors whose mask rows take the
                     // embeddings of the current drafts (iterative denoising)
  __host__ __device__ int rows() const { return kind == PASS_DRAFT ? RM + A * B : B * Kx; }
  __host__ __device__ int tokens_per_seq() const { return A + Kx; }
};

struct RowInfo {
  int b, t, pos, limit, is_mask, pad;
};

// Physical row r -> (sequence, token index within the sequence's rows
// [anchor first], absolute position, last visible cache slot, mask-row flag,
// padding flag).
__device__ __forceinline__ RowInfo row_info(const PassInfo& P, int r) {
  RowInfo ri;
  ri.pad = 0;
  if (P.kind == PASS_DRAFT) {
    if (r >= P.RM) {
      ri.b = r - P.RM; ri.t = 0; ri.pos = P.len[ri.b]; ri.limit = ri.pos; ri.is_mask = 0;
    } else if (r < P.B * P.Kx) {
      ri.b = r / P.Kx;
      int i = r - ri.b * P.Kx;
      ri.t = P.A + i;
      int n = P.len[ri.b];
      ri.pos = n + 1 + i; ri.limit = n; ri.is_mask = 1;
    } else {
      ri.b = 0; ri.t = 0; ri.pos = 0; ri.limit = -1; ri.is_mask = 0; ri.pad = 1;
    }
  } else {
    ri.b = r / P.Kx;
    int i = r - ri.b * P.Kx;
    ri.t = i;
    ri.pos = (P.kind == PASS_VERIFY ? P.len[ri.b] + 1 : P.p0) + i;
    ri.limit = ri.pos; ri.is_mask = 0;
  }
  return ri;
}

__host__ __device__ __forceinline__ int row_of(const PassInfo& P, int b, int t) {
  if (P.kind == PASS_DRAFT) return t < P.A ? P.RM + b : b * P.Kx + (t - P.A);
  return b * P.Kx + t;
}

// Column of key j (0..63) inside a 64-key V tile stored transposed
// ([head_dim][64]): within each 32-key group the 4-key runs are interleaved
// so that one 16-byte LDS read gives a lane the 8 keys its MFMA B-operand
// slot needs (keys q*4..q*4+3 and 16+q*4..16+q*4+3 for lane group q).
__host__ __device__ __forceinline__ int vt_col(int j) {
  int g = j >> 5, k = j & 31;
  return g * 32 + ((k & 15) >> 2) * 8 + (k >> 4) * 4 + (k & 3);
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += ((u >> 16) & 1u) + 0x7FFFu;        // round to nearest even (inputs are finite)
  return (uint16_t)(u >> 16);
}

// ----------------------------------------------------------- launchers
// common kernels
void launch_pack_bf16(const uint16_t* src, int N, int K, void* dst, int nb_off, int nb_stride,
                      hipStream_t s);
void launch_stream_read(const void* buf, uint64_t bytes, uint32_t* out, int nwg, hipStream_t s);
void launch_embed(const PassInfo& P, const int32_t* anchor_tok, const int32_t* block_tok,
                  int block_ld, const void* embed, const void* mask_emb, int V, int d, bool bf16,
                  float* h, hipStream_t s);
// h[r] += ((p0 + p1) + ... + p7)[r] (nslices 8, part [8][rows][d] with slice
// stride ps; nslices 0: no residual), then out[r] = bf16(RMSNorm(h[r]) * g).
// Padding rows of a draft pass are left alone.
void launch_resid_norm_bf16(const PassInfo& P, float* h, int d, const float* part, size_t ps,
                            int nslices, const uint16_t* gain, float eps, uint16_t* out,
                            hipStream_t s);
void launch_rmsnorm(const float* h, int rows, int d, const void* gain, bool bf16, float eps,
                    void* out, hipStream_t s);
void launch_qkv_post(const PassInfo& P, const float* qkv, int hq, int hkv, int hd,
                     const void* qn, const void* kn, const void* dqn, const void* dkn, bool bf16,
                     float eps, const float* rope, void* q_out, void* kc, void* vc, int cap,
                     void* ks, void* vs, int kpad, hipStream_t s);
void launch_lm_reduce(const float2* part, int rows, int nparts, const PassInfo& P, int K,
                      int32_t* drafts, int32_t* ar_tokens, int32_t* pending, hipStream_t s);
// K drafts per sequence, stored with row stride ld (drafts [B][ld], ar [B][ld + 1])
void launch_accept(int B, int K, int ld, const int32_t* drafts, const int32_t* ar,
                   int32_t* accept_len, hipStream_t s);
// ld: row stride of drafts [B][ld] and ar [B][ld + 1]
void launch_commit(int B, int ld, const int32_t* accept_len, const int32_t* ar,
                   const int32_t* drafts, int32_t* seq_len, int32_t* pending,
                   int32_t* commit_start, int32_t* out_tokens, int32_t* out_off, hipStream_t s);
// seq_len[b] = prompt length - 1 (the length clamped to [1, pmax]) and
// last_tok[b] = the prompt's last token
void launch_prefill_tail(int B, const int32_t* tokens, int ld, const int32_t* plen_dev, int pmax,
                         int32_t* seq_len, int32_t* last_tok, hipStream_t s);
void launch_len_add(int B, int32_t* seq_len, int add, hipStream_t s);

// GEMMs.  Y = X . W^T over rows [0, M) of X (row stride ldx elements).
enum Epilogue { EP_STORE = 0, EP_RESID = 1, EP_SWIGLU = 2, EP_ARGMAX = 3, EP_QKV = 4 };
struct GemmOut {                // fp32 path
  int ep;
  float* y; int ldy;            // EP_STORE / EP_RESID (fp32)
  void* act; int ldact;         // EP_SWIGLU
  float2* part;                 // EP_ARGMAX partials [M][1]
  float* logits; int ldl;       // optional logits tap (EP_ARGMAX)
};

// bf16 path: one launch covers GEMM rows [0, M) = pass rows [row0, row0+M).
// The bf16 activations that feed the GEMMs (RMSNorm output, attention
// output, SwiGLU product) are stored in MFMA fragment order: row tiles of
// 16 rows, k-blocks of 32 columns, and within a (tile, k-block) the 64
// lanes' 16-byte B-operand pieces in lane order (lane = 16 * (k / 8 % 4) +
// row % 16), so a wave loads a fragment as 1 KB of contiguous memory.  kb =
// columns / 32.  Element offset of (row r, column k):
__host__ __device__ __forceinline__ size_t frag_off(int r, int k, int kb) {
  return ((size_t)(r >> 4) * kb + (k >> 5)) * 512 + (size_t)(((((k >> 3) & 3) << 4) | (r & 15)) * 8 + (k & 7));
}

struct GemmArgs {
  const u32x4_t* W;             // packed weight (16x32 MFMA fragments)
  int M, K, N, row0;
  const u32x4_t* W2; int M2, row02;   // optional second segment (other weights and rows)
  int gy0;                      // row blocks of the first segment (set by the launcher)
  int gyt;                      // row blocks of both segments (set by the launcher)
  int flat;                     // 1-D grid over (column group, row block) (set by the launcher)
  const uint16_t* X; int ldx;   // bf16 input, fragment order (K / 32 k-blocks; ldx = K)
  // split-K partials [8][M][N] and completion counters (zero between launches)
  float* part; unsigned* cnt;
  int ep;
  float* y; int ldy;                                  // EP_RESID (wide: y += result)
  float* rpart; size_t rps;     // EP_RESID / EP_QKV split-K: slice partials [8][rows][N] (slice stride rps)
  uint16_t* act; int ldact;                            // EP_SWIGLU
  PassInfo P; int hq, hkv; float eps;                  // EP_QKV (and EP_ARGMAX row mapping)
  const uint16_t* qn; const uint16_t* kn; const uint16_t* dqn; const uint16_t* dkn;
  const float2* rope; uint16_t* q_out; uint16_t* kc; uint16_t* vc; int cap;
  uint16_t* ks; uint16_t* vs; int kpad;
  float2* amax; float* logits; int ldl; int Kb;       // EP_ARGMAX
  int32_t* drafts; int32_t* ar; int32_t* pending;
  int tnrb, ttb, tng;           // row-split launches: row blocks, row tiles per block, column groups (set by the launcher)
  int defer_finish;             // EP_QKV launches that write slice partials: the caller runs the finish kernel
};
void launch_gemm_bf16(const GemmArgs& a, hipStream_t s);
// QKV finish over the slice partials of one or two earlier split launches
// (rows [0, M) from row0, [M, M + M2) from row02)
void launch_qkv_finish_bf16(const GemmArgs& a, hipStream_t s);
// Profiling: the next bf16 GEMM kernel launched from this host thread
// records start / stop itself (hipExtLaunchKernel); pending until taken.
void gemm_time_next_launch(hipEvent_t start, hipEvent_t stop);
bool gemm_time_pending();
int gemm_bf16_groups(int N);
// 0, or the K slices whose partials an EP_RESID launch of these rows leaves
// for the residual + RMSNorm kernel
int gemm_bf16_split_slices(int M, int M2, int N, int ep);
// whether a one-segment launch of M rows takes the row-split form
bool gemm_bf16_rows_form(int M, int N, int ep);
// fp32: W canonical row-major [N][K] (for SwiGLU: gate at W, up at W2).
void launch_gemm_f32(const float* W, const float* W2, const float* X, int ldx, int M, int K,
                     int N, const GemmOut& o, hipStream_t s);

// Attention.  q [rows][hq][hd] (model dtype); cache layer base pointers.
struct AttnArgs {
  PassInfo P;
  const void* q;
  const void* kc; const void* vc; int cap;
  const void* ks; const void* vs; int kpad;   // block scratch (draft passes)
  int hq, hkv, hd;
  int sc;           // keys per chunk (multiple of 64)
  int nc;           // cache chunks
  int qr_max;       // q-rows per (sequence, kv head) capacity of the partial buffers
  float* opart;     // [B][hkv][nc+1][qr_max][hd]
  float* ml;        // [B][hkv][nc+1][qr_max][2]
  void* out;        // model dtype: [rows][hq*hd], or fragment order when out_kb > 0
  int out_kb;       // bf16 output in fragment order with out_kb = hq*hd/32 k-blocks (0: row-major)
  void* tap; int tap_rows;   // optional attention-output tap for this layer
  float* tap32; int tap32_rows;   // optional fp32 tap of the attention output before rounding
  int fixed_ctx;    // >= 0: microbenchmark mode, every row sees cache [0, fixed_ctx)
  int block_len;    // keys in the block scratch
  int active_chunks;  // upper bound on the cache chunks a sequence of the pass reaches
  int tpw;          // query tiles per wave, 1 or 2 (0: the launcher chooses from the grid size)
};
void launch_attention_bf16(const AttnArgs& a, hipStream_t s);

// Sampling at T > 0 (k_sample.hip).  dlogits / dstats: the draft pass's
// logits [rows][V] and per-row (max, weight sum); vlogits / vstats: the
// verify pass's; RM: the draft pass's first anchor row.
struct SampleArgs {
  float T;
  uint64_t seed;
  uint32_t step;
  int V, RM;
  const float* dlogits; const float* vlogits;
  const float2* dstats; const float2* vstats;
};
// per row of pass P: (max, weight sum) into stats; the mask rows of a draft
// pass also draw their drafts (drafts [B][Kb])
void launch_sample_rows(const SampleArgs& s, const PassInfo& P, const float* logits, int ld,
                        float2* stats, int32_t* drafts, int Kb, hipStream_t st);
// the first generated token after a prefill: a sample of each sequence's
// anchor row RM + b (its stats already computed)
void launch_sample_first(const SampleArgs& s, int B, int RM, const float* logits,
                         const float2* stats, int32_t* pending, hipStream_t st);
// acceptance of the K drafts and the final token, per sequence: accept_len,
// ar[b][0..m) = the accepted drafts, ar[b][m] = the final token
void launch_spec_accept(const SampleArgs& s, int B, int K, int ld_tok, const int32_t* drafts,
                        int32_t* ar, int32_t* accept_len, hipStream_t st);
// number of query row groups of a pass: a workgroup's four waves own tpw
// 16-row query tiles each
__host__ __device__ inline int attn_row_groups(int qr, int tpw) {
  return ((qr + 15) / 16 + 4 * tpw - 1) / (4 * tpw);
}
void launch_attention_f32(const AttnArgs& a, hipStream_t s);
