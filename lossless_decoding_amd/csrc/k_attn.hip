// Block attention over the shared KV cache (the draft pass's anchor + mask
// rows, the verify pass's causal rows, prefill rows).
//
// bf16 path.  A workgroup handles (key chunk, KV head, sequence, group of
// 16-row query tiles); the query rows of a sequence are its tokens x
// the G query heads of the KV head, so each 64-key K/V tile staged in LDS
// serves the whole GQA group.  A wave owns one or two query tiles.
// MFMA: S^T = K . Q^T (keys x rows) and O^T = V^T . P^T (dims x rows), so a
// lane always holds one query row and the softmax statistics stay in-lane.
// Softmax in fp32 with a base-2 exponent against a per-row reference that is
// raised only when a tile's scores exceed it by more than 2^8.  K/V tiles go
// from memory straight into a five-slot LDS ring, three tile halves ahead of
// the one computed.  Chunks are SC keys aligned to absolute cache positions;
// the sequence's last chunk also streams the draft block's keys, after its
// cache keys.  Each chunk writes its partial (reference, sum, unnormalised
// output) and the merge kernel combines a row's partials in increasing chunk
// order.  An AR row's result therefore depends only on which keys it sees,
// never on the other rows of the pass or the launch shape: fully masked
// tiles and chunks are exact no-ops, masked keys are removed by selection
// (never by multiplying stale values), and keys past the pass's last written
// slot are zeroed when staged.  A mask row also depends on the launch's
// query tiles per wave: with two the draft block's keys are folded into the
// last chunk's partial, with one they form a partial of their own (the
// library fixes that choice per context for draft passes).
//
// fp32 path: one wave per (row, query head), keys in order (check models).
#include "internal.h"

// Staged tiles in LDS: K as 64 key rows of 256 bytes, V^T as 128 dimension
// rows of 128 bytes (64 keys in the cache's column order).  The 16-byte units
// of a row are XOR-permuted by the row index (K: unit ^ (key & 15), V^T:
// unit ^ (dim & 7)), which keeps the MFMA fragment reads (16 rows x 16 bytes
// per group of lanes) free of LDS bank conflicts; padded rows would block the
// direct memory-to-LDS loads, which fill 1 KB of LDS in lane order.
__device__ __forceinline__ int k_lds_off(int key, int cu) { return key * 256 + ((cu ^ (key & 15)) << 4); }
__device__ __forceinline__ int v_lds_off(int d, int ku) { return d * 128 + ((ku ^ (d & 7)) << 4); }

__device__ __forceinline__ bf16x8_t ld_bf16x8(const uint16_t* p) {
  uint4 v = *(const uint4*)p;
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// x, as a value the compiler cannot see through (no instruction): keeps it
// from precomputing and holding values derived from x across a loop.  The
// register constraint exists only in the device pass.
__device__ __forceinline__ int opaque(int x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(x));
#endif
  return x;
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

// A row's softmax reference m (base 2) is raised only when a tile holds a
// score above m + REF_SLACK; otherwise the tile's weights 2^(s - m) stay
// below 2^REF_SLACK and are used against the old reference.  The decision is
// taken per row from that row's own scores, so the arithmetic a row sees is
// still a function of its keys alone.
#define REF_SLACK 8.0f
// a lane's eight keys of a half tile drop the low P term when their weights
// sum to at most this share of the lane's running sum
#define LO_SKIP 0.125f

template <int N> struct IntC { static constexpr int value = N; };

// LDS ring of ATT_SLOTS 16 KB slots.  A 64-key tile is two units, its K
// (64 key rows of 256 bytes) and its V^T (128 dimension rows of 128 bytes);
// unit u (K of tile i = 2i, V^T = 2i + 1) lives in slot u % ATT_SLOTS.  With
// five slots three units are in flight while a tile is computed, and two
// workgroups (80 KB each) share a compute unit's 160 KB.
#define ATT_SLOTS 5

// The kernel body, for TPW query tiles per wave (four waves per workgroup,
// two workgroups per compute unit), with cache policy KVPOL on the K/V tile
// loads (0: default; 2: non-temporal, for launches in which every key tile
// is read by one workgroup only -- a single row group -- so that the
// streamed keys do not hold L2 lines).  It is a device template behind plain
// kernels, so only the device pass instantiates it.
template <int TPW, int KVPOL>
__device__ __forceinline__ void attn_bf16_body(const AttnArgs& a) {
  constexpr int NW = 4;
  // each 16 KB unit is 16 one-kilobyte loads, LPU of them per wave
  constexpr int LPU = 16 / NW;
  // one array per slot, so the compiler sees that loads into one slot and
  // reads of another do not alias (no wait for in-flight loads)
  __shared__ __attribute__((aligned(16))) uint16_t sR0[8192];
  __shared__ __attribute__((aligned(16))) uint16_t sR1[8192];
  __shared__ __attribute__((aligned(16))) uint16_t sR2[8192];
  __shared__ __attribute__((aligned(16))) uint16_t sR3[8192];
  __shared__ __attribute__((aligned(16))) uint16_t sR4[8192];
  auto slot = [&](auto sc) __attribute__((always_inline)) -> uint16_t* {
    constexpr int S = decltype(sc)::value % ATT_SLOTS;
    if constexpr (S == 0) return sR0;
    else if constexpr (S == 1) return sR1;
    else if constexpr (S == 2) return sR2;
    else if constexpr (S == 3) return sR3;
    else return sR4;
  };
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
  const PassInfo& P = a.P;
  const int T = a.fixed_ctx >= 0 ? P.Kx : P.tokens_per_seq();
  const int G = a.hq / a.hkv;
  const int QR = T * G;
  const int NRT = (QR + 15) >> 4;
  const int NRG = attn_row_groups(QR, TPW);
  // 1-D grid over (chunk, KV head, sequence x row group), chunk fastest.
  // The draft block's keys (at most one tile) are streamed by the
  // sequence's last chunk after its cache keys (chunk 0 when there are no
  // cache keys) when the launch has two query tiles per wave (many
  // workgroups: one partial fewer per row, no short block workgroups in a
  // second round); with one tile per wave (a launch that fits in one round)
  // by a block workgroup of their own, chunk index nc, in parallel.
  constexpr bool FOLD = TPW == 2;
  const int ncol = FOLD ? a.nc : a.nc + 1;
  const int c = blockIdx.x % ncol;
  const int g = (blockIdx.x / ncol) % a.hkv;
  const int zz = blockIdx.x / (ncol * a.hkv);
  const int b = zz / NRG, rg = zz - b * NRG;
  const int hd = 128;
  const int H = a.hq * hd;

  // which chunks take part: every chunk up to the sequence's last visible
  // slot, and the block
  const bool has_blk = a.block_len > 0 && (a.fixed_ctx >= 0 || (P.kind == PASS_DRAFT && P.Kx > 0));
  const SeqLimits L = seq_limits(a, b);
  const int lastk = L.maxlim < a.cap - 1 ? L.maxlim : a.cap - 1;
  const int nch = lastk >= 0 ? lastk / a.sc + 1 : 0;
  const int c_last = nch > 0 ? nch - 1 : 0;
  const bool blk_wg = !FOLD && c == a.nc;                                  // block keys only
  if (blk_wg ? !has_blk : (c > c_last || (nch == 0 && !(FOLD && has_blk)))) return;
  const int k_begin = blk_wg ? 0 : c * a.sc;
  const int k_end = (blk_wg || nch == 0) ? k_begin : min(k_begin + a.sc, lastk + 1);   // cache keys
  const int nct = (k_end - k_begin + 63) >> 6;                             // cache tiles
  const int ntot = nct + ((has_blk && (blk_wg || (FOLD && c == c_last))) ? 1 : 0);   // + block tile

  // This wave's query tiles rt0 .. rt0 + tpw - 1 (B operands of
  // S^T = K.Q^T); lane row qr = rt*16 + lr.  A padding row (qr >= QR) gets a
  // zero query that sees every key: it computes harmless values that are
  // never stored.  Which wave computes a row changes none of its arithmetic.
  const int rt0 = (rg * NW + wave) * TPW;
  const int nt = rt0 >= NRT ? 0 : (TPW == 2 && rt0 + 1 < NRT ? 2 : 1);   // uniform per wave
  bf16x8_t qf[2][4];
  int lim[2], seesb[2];
  floatx4_t oacc[2][8];
  float mref[2], thr[2], lsum[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    mref[t] = -INFINITY; thr[t] = -INFINITY; lsum[t] = 0.f;
    lim[t] = 0x7fffffff; seesb[t] = 1;
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[t][db] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    const int qr = (rt0 + t) * 16 + lr;
    if (t < nt && qr < QR) {
      const int tk = qr / G, hh = g * G + (qr - tk * G);
      const int r = row_of(P, b, tk);
      token_view(a, L, tk, lim[t], seesb[t]);
      const uint16_t* qp = (const uint16_t*)a.q + (size_t)r * H + hh * hd + lq * 8;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) qf[t][ds] = ld_bf16x8(qp + ds * 32);
    } else {
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) qf[t][ds] = bf16x8_t{};
    }
  }
  const int lmin = nt == 2 ? min(lim[0], lim[1]) : lim[0];

  const uint16_t* kbase = (const uint16_t*)a.kc + ((size_t)b * a.hkv + g) * a.cap * hd;
  const uint16_t* vbase = (const uint16_t*)a.vc + ((size_t)b * a.hkv + g) * a.cap * hd;   // tiles of 64*hd
  const uint16_t* kblk = (const uint16_t*)a.ks + ((size_t)b * a.hkv + g) * a.kpad * hd;
  const uint16_t* vblk = (const uint16_t*)a.vs + ((size_t)b * a.hkv + g) * hd * a.kpad;
  const float sl2 = 1.4426950408889634f / sqrtf((float)hd);

  // Tiles go from memory straight into LDS (buffer loads with an LDS
  // destination): per tile each wave moves 4 KB of K and 4 KB of V^T, one
  // kilobyte per instruction (64 lanes x 16 bytes, in lane order), each lane
  // fetching the piece that the XOR permutation puts at its position.  The
  // descriptors cover one tile: K pieces past the last key, V^T pieces past
  // the tile and every piece of a tile past the last read as zero without
  // touching memory.  V^T columns of keys past the end within a partial tile
  // hold whatever memory holds there; they are zeroed in LDS.  Tile i < nct
  // is the cache tile at key k_begin + 64 i; tile nct is the draft block
  // (K rows [kpad][128], V^T [128][kpad] in the same column order).
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  int koff[LPU], voff[LPU];
#pragma unroll
  for (int j = 0; j < LPU; ++j) {
    const int key = (wv * LPU + j) * 4 + (lane >> 4);
    koff[j] = key * 256 + (((lane & 15) ^ (key & 15)) << 4);   // unit (lane & 15) ^ (key & 15) of the key
    const int d = (wv * LPU + j) * 8 + (lane >> 3);
    voff[j] = d * 128 + (((lane & 7) ^ (d & 7)) << 4);         // unit (lane & 7) ^ (d & 7) of the row
  }
  auto issue_k = [&](uint16_t* dst, int i) __attribute__((always_inline)) {
    const uint16_t* src = kbase;
    int nk = 0;
    if (i < nct) {
      const int kt = k_begin + i * 64;
      src = kbase + (size_t)kt * hd;
      nk = min(64, k_end - kt);
    } else if (i < ntot) {
      src = kblk;
      nk = a.block_len;
    }
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, nk * hd * 2, 0x00020000);
#pragma unroll
    for (int j = 0; j < LPU; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(dst + (wv * LPU + j) * 512), 16, koff[j], 0, 0,
          KVPOL);
  };
  // V^T: a cache tile is 128 rows of 64 keys; the block's rows are kpad
  // keys long (pieces past kpad belong to the next row; they are zeroed in
  // LDS with the keys past block_len).  One load sequence for both, so the
  // compiler tracks each slot's loads as one group.
  auto issue_v = [&](uint16_t* dst, int i) __attribute__((always_inline)) {
    const bool bt = i >= nct && i < ntot;                      // uniform
    const uint16_t* src = bt ? vblk : vbase + (size_t)((k_begin >> 6) + (i < nct ? i : 0)) * 64 * hd;
    const int bytes = i >= ntot ? 0 : (bt ? hd * a.kpad * 2 : 64 * hd * 2);
    const int row_extra = bt ? a.kpad * 2 - 128 : 0;         // row length - 128 bytes
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, bytes, 0x00020000);
#pragma unroll
    for (int j = 0; j < LPU; ++j) {
      const int d = (wv * LPU + j) * 8 + (lane >> 3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(dst + (wv * LPU + j) * 512), 16,
          voff[j] + d * row_extra, 0, 0, KVPOL);
    }
  };
  // zero the V^T columns of keys >= nvalid (the last, partial tile)
  auto zero_v = [&](uint16_t* V, int nvalid) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 16 / NW; ++m) {
      const int u = opaque(tid + m * NW * 64);                 // 16-byte unit of the tile (rare path)
      const int d = u >> 3, ku = (u & 7) ^ (d & 7);
      uint4 v = *(uint4*)(V + u * 8);
      uint16_t e[8];
      __builtin_memcpy(e, &v, 16);
#pragma unroll
      for (int x = 0; x < 8; ++x)
        if (vt_key(ku * 8 + x) >= nvalid) e[x] = 0;
      __builtin_memcpy(&v, e, 16);
      *(uint4*)(V + u * 8) = v;
    }
  };
  // fragment offsets (bytes) of this lane: K for ds = 0..3 (+ kb*4096),
  // V^T for ks = 0..1 (+ db*2048)
  int kfo[4], vfo[2];
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) kfo[ds] = k_lds_off(lr, ds * 4 + lq);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) vfo[ks] = v_lds_off(lr, ks * 4 + lq);

  // The tile's work for the wave's NT query tiles.  Every K and V^T
  // fragment read from LDS feeds one MFMA per query tile.
  auto compute = [&](const uint16_t* sK, const uint16_t* sV, auto ntc, int kt, int nvalid, bool bt)
      __attribute__((always_inline)) {
    constexpr int NT = decltype(ntc)::value;
    const char* sKb = (const char*)sK;
    const char* sVb = (const char*)sV;
    // fresh copies of the lane's fragment offsets each step, so the slot
    // addresses are formed here (one add each) rather than kept in
    // registers for all five slots
    int ko[4], vo[2];
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) ko[ds] = opaque(kfo[ds]);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) vo[ks] = opaque(vfo[ks]);
    // S^T for 4 blocks of 16 keys
    floatx4_t s[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[t][kb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    // dimension steps outer, so consecutive MFMAs use different accumulators
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8_t kf = ld_bf16x8((const uint16_t*)(sKb + kb * 4096 + ko[ds]));
#pragma unroll
        for (int t = 0; t < NT; ++t)
          s[t][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[t][ds], s[t][kb], 0, 0, 0);
      }
    // Visibility: when every key of the tile is visible to every row of the
    // wave (the common case at long context) nothing is masked; otherwise
    // invisible keys get the score -inf.
    const bool all_vis = !bt && nvalid == 64 && __all(kt + 63 <= lmin);
    if (!all_vis) {
      const int lq4 = opaque(lq * 4);                          // (keeps no per-key constants live)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kl = kb * 16 + lq4 + i;
            const bool ok = kl < nvalid && (bt ? seesb[t] != 0 : (kt + kl) <= lim[t]);
            s[t][kb][i] = ok ? s[t][kb][i] : -INFINITY;
          }
    }
    // Reference update.  A row needs one when some lane of the row (its
    // four lanes hold lanes lr, lr+16, lr+32, lr+48) has a scaled score
    // above m + REF_SLACK; the ballot, folded to 16 row bits, says which.
    // Only then the row maximum is formed across the lanes and the row's
    // o and l are rescaled (a row that needs none keeps m and is multiplied
    // by exactly 1).
    float lm[NT];
    uint32_t rowbits[NT];
    uint32_t anyrow = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[t][kb][i]);
      lm[t] = mx;
      const uint64_t bal = __ballot(mx * sl2 > thr[t]);
      rowbits[t] = (uint32_t)(bal | (bal >> 16) | (bal >> 32) | (bal >> 48)) & 0xffffu;
      anyrow |= rowbits[t];
    }
    if (anyrow) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (rowbits[t] == 0) continue;
        float rm = lm[t];
        rm = fmaxf(rm, __shfl_xor(rm, 16, 64));
        rm = fmaxf(rm, __shfl_xor(rm, 32, 64));
        const bool rn = (rowbits[t] >> lr) & 1u;
        const float mnew = rn ? fmaxf(mref[t], rm * sl2) : mref[t];
        // m = -inf (nothing seen yet): 2^-inf = 0, and o, l are still 0
        const float alpha = rn ? __builtin_amdgcn_exp2f(mref[t] - mnew) : 1.f;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          oacc[t][db][0] *= alpha; oacc[t][db][1] *= alpha;
          oacc[t][db][2] *= alpha; oacc[t][db][3] *= alpha;
        }
        lsum[t] *= alpha;
        mref[t] = mnew;
        thr[t] = mnew + REF_SLACK;
      }
    }
    // Weights p = 2^(s * scale - m), one fused multiply-add and v_exp_f32
    // each (arguments <= REF_SLACK; results below 2^-126 are negligible
    // weights and flush to 0).  A row whose m is still -inf has only -inf
    // scores so far, so its p are 0.  l is summed per lane, eight keys at a
    // time in a fixed tree, and across the row's lanes once, at the end.
    // P enters the P.V product as hi = bf16(p) and, where it matters,
    // lo = bf16(p - hi) (p - hi is exact in fp32): about 16 significant bits
    // of p instead of 8.  lo is dropped for a lane's eight keys of a half
    // tile when their weights sum to at most LO_SKIP of the lane's running
    // sum l; hi alone then carries them (relative error <= 2^-9 on a small
    // share of the total).  The decision depends only on the row's own keys
    // and position-aligned tiles, and a dropped lo is an exact zero in the
    // product, so the lo MFMAs are issued only when some lane keeps lo.
    // Done in two halves of 32 keys (kb 0-1, then kb 2-3), so only half of
    // P is live at a time; each accumulator sums its terms in the same order
    // (keys 0-31 hi, lo, then keys 32-63 hi, lo).
    float mr[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) mr[t] = mref[t] == -INFINITY ? 0.f : mref[t];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float pv[NT][8];
      bool keep[NT];
      bool any_keep = false;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pv[t][kh * 4 + i] =
                __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][ks * 2 + kh][i], sl2, -mr[t]));
        const float ts = ((pv[t][0] + pv[t][1]) + (pv[t][2] + pv[t][3])) +
                         ((pv[t][4] + pv[t][5]) + (pv[t][6] + pv[t][7]));
        keep[t] = ts > lsum[t] * LO_SKIP;
        lsum[t] += ts;
        any_keep = any_keep || keep[t];
      }
      bf16x8_t pf[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 8; ++j) pf[t][j] = (__bf16)pv[t][j];
      // two dimension blocks at a time, hi terms before lo terms, so an
      // MFMA never waits on the one just issued (same per-accumulator order)
      if (__any(any_keep)) {
        bf16x8_t pl[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            pl[t][j] = keep[t] ? (__bf16)(pv[t][j] - (float)pf[t][j]) : (__bf16)0.f;
#pragma unroll
        for (int db = 0; db < 8; db += 2) {
          const bf16x8_t vf0 = ld_bf16x8((const uint16_t*)(sVb + db * 2048 + vo[ks]));
          const bf16x8_t vf1 = ld_bf16x8((const uint16_t*)(sVb + (db + 1) * 2048 + vo[ks]));
#pragma unroll
          for (int t = 0; t < NT; ++t)
            oacc[t][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf0, pf[t], oacc[t][db], 0, 0, 0);
#pragma unroll
          for (int t = 0; t < NT; ++t)
            oacc[t][db + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf1, pf[t], oacc[t][db + 1], 0, 0, 0);
#pragma unroll
          for (int t = 0; t < NT; ++t)
            oacc[t][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf0, pl[t], oacc[t][db], 0, 0, 0);
#pragma unroll
          for (int t = 0; t < NT; ++t)
            oacc[t][db + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf1, pl[t], oacc[t][db + 1], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int db = 0; db < 8; db += 2) {
          const bf16x8_t vf0 = ld_bf16x8((const uint16_t*)(sVb + db * 2048 + vo[ks]));
          const bf16x8_t vf1 = ld_bf16x8((const uint16_t*)(sVb + (db + 1) * 2048 + vo[ks]));
#pragma unroll
          for (int t = 0; t < NT; ++t)
            oacc[t][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf0, pf[t], oacc[t][db], 0, 0, 0);
#pragma unroll
          for (int t = 0; t < NT; ++t)
            oacc[t][db + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf1, pf[t], oacc[t][db + 1], 0, 0, 0);
        }
      }
    }
  };

  // One tile step: wait until the tile's two units are in LDS (own loads:
  // only the next tile's K, issued one step earlier, may still be in
  // flight; then the barrier for everyone's, which also ends every wave's
  // reads of the previous tile's slots), zero V^T columns past the end,
  // start V^T of the next tile and K of the one after into the two freed
  // slots, compute.  Every wave runs the same steps with the number of query
  // tiles it owns.  Units past the end are size-0 loads (zeros, no memory
  // access); all loads have landed before the workgroup ends.
  // The step barrier is the hardware barrier alone.  A workgroup fence
  // (__syncthreads) would also wait for every load still filling a later
  // slot; the explicit wait before it covers exactly this tile's units.
  // The empty asm statements keep the compiler from moving LDS accesses
  // across it (they emit nothing); the wait before it also takes lgkmcnt to
  // 0, so no wave still has a read of the previous tile's slots in flight
  // when another wave starts loads into them.
  auto step_barrier = []() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Launches with few workgroups (one query tile per wave; B = 1 decode)
  // have chunks of one or two tiles: there a plain two-stage schedule
  // (slots 0-1 and 2-3) loads whole tiles, waits for all loads, and loads
  // no tile past the end.
  auto run2 = [&](auto ntc) __attribute__((always_inline)) {
    auto step = [&](auto s1c, int i) __attribute__((always_inline)) {
      constexpr int S1 = decltype(s1c)::value;
      const bool bt = i >= nct;                                // the block tile
      const int kt = bt ? 0 : k_begin + i * 64;
      const int nvalid = bt ? a.block_len : min(64, k_end - kt);
      __builtin_amdgcn_s_waitcnt(0x0f70);                      // vmcnt(0)
      __syncthreads();
      if (nvalid < 64) {
        zero_v(slot(IntC<2 * S1 + 1>{}), nvalid);
        __syncthreads();
      }
      if (i + 1 < ntot) {
        issue_k(slot(IntC<2 - 2 * S1>{}), i + 1);
        issue_v(slot(IntC<3 - 2 * S1>{}), i + 1);
      }
      if constexpr (decltype(ntc)::value > 0)
        compute(slot(IntC<2 * S1>{}), slot(IntC<2 * S1 + 1>{}), ntc, kt, nvalid, bt);
    };
    issue_k(slot(IntC<0>{}), 0);
    issue_v(slot(IntC<1>{}), 0);
    for (int i = 0; i < ntot; i += 2) {
      step(IntC<0>{}, i);
      if (i + 1 < ntot) step(IntC<1>{}, i + 1);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);                        // vmcnt(0)
  };
  auto run = [&](auto ntc) __attribute__((always_inline)) {
    if constexpr (TPW == 1) {
      run2(ntc);
      return;
    }
    // tile i: K in slot (2i) % 5 = S0, V^T in S0 + 1; the freed slots of
    // tile i - 1 are S0 + 3 and S0 + 4 (mod 5)
    auto step = [&](auto s0c, int i) __attribute__((always_inline)) {
      constexpr int S0 = decltype(s0c)::value;
      const bool bt = i >= nct;                                // the block tile
      const int kt = bt ? 0 : k_begin + i * 64;
      const int nvalid = bt ? a.block_len : min(64, k_end - kt);
      __builtin_amdgcn_s_waitcnt(0x0070 | LPU);                // vmcnt(LPU) lgkmcnt(0)
      step_barrier();
      if (nvalid < 64) {
        zero_v(slot(IntC<S0 + 1>{}), nvalid);
        __syncthreads();
      }
      issue_v(slot(IntC<S0 + 3>{}), i + 1);
      issue_k(slot(IntC<S0 + 4>{}), i + 2);
      if constexpr (decltype(ntc)::value > 0)
        compute(slot(IntC<S0>{}), slot(IntC<S0 + 1>{}), ntc, kt, nvalid, bt);
    };
    issue_k(slot(IntC<0>{}), 0);
    issue_v(slot(IntC<1>{}), 0);
    issue_k(slot(IntC<2>{}), 1);
    // five tiles per round bring the slots back to the start; every step
    // issues exactly 2 LPU loads per wave after its wait, so at a step's
    // wait the last LPU are the next tile's K
    for (int i = 0; i < ntot; i += 5) {
      step(IntC<0>{}, i);
      if (i + 1 < ntot) step(IntC<2>{}, i + 1);
      if (i + 2 < ntot) step(IntC<4>{}, i + 2);
      if (i + 3 < ntot) step(IntC<1>{}, i + 3);
      if (i + 4 < ntot) step(IntC<3>{}, i + 4);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);                        // vmcnt(0)
  };
  if (TPW == 2 && nt == 2) run(IntC<TPW == 2 ? 2 : 1>{});
  else if (nt == 1) run(IntC<1>{});
  else run(IntC<0>{});

  // ---- partials of this chunk: opart[((b*hkv+g)*(nc+1)+c)*qr_max + qr][d],
  // ml[...][2] = (m, l); l is summed over the row's four lanes in a fixed
  // butterfly
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t >= nt) break;
    float l = lsum[t];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int qr = (rt0 + t) * 16 + lr;
    if (qr < QR) {
      const size_t pi = ((size_t)(b * a.hkv + g) * (a.nc + 1) + c) * a.qr_max + qr;
      float* op = a.opart + pi * hd;
#pragma unroll
      for (int db = 0; db < 8; ++db) *(floatx4_t*)(op + db * 16 + lq * 4) = oacc[t][db];
      if (lq == 0) {
        a.ml[pi * 2 + 0] = mref[t];
        a.ml[pi * 2 + 1] = l;
      }
    }
  }
}

// one query tile per wave (launches with few workgroups), two per wave
__global__ __launch_bounds__(256, 2) void k_attn_bf16_t1(AttnArgs a) { attn_bf16_body<1, 0>(a); }
__global__ __launch_bounds__(256, 2) void k_attn_bf16_t2(AttnArgs a) { attn_bf16_body<2, 0>(a); }
// the same with non-temporal K/V loads (launches of a single row group)
__global__ __launch_bounds__(256, 2) void k_attn_bf16_t1_stream(AttnArgs a) { attn_bf16_body<1, 2>(a); }
__global__ __launch_bounds__(256, 2) void k_attn_bf16_t2_stream(AttnArgs a) { attn_bf16_body<2, 2>(a); }

// Combine the chunk partials of one (row, query head); one wave each, four
// per block.  Phase 1: the maximum M of the chunk maxima the row sees.
// Phase 2: l = sum_c l_c 2^(m_c - M) and o = sum_c o_c 2^(m_c - M), summed
// in increasing chunk order.  All loads of a phase are independent, so the merge costs two
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
  // the row folds the partials of the chunks it sees; the draft block's
  // keys are inside the sequence's last chunk (chunk 0 without cache keys)
  // after a two-tile launch, in partial nc (folded last) after a one-tile one
  const int nrow = limit >= 0 ? limit / a.sc + 1 : 0;
  const bool blocked = sees && has_blk;
  const bool folded = a.tpw == 2;
  const int ntot = folded ? (nrow > 0 ? nrow : (blocked ? 1 : 0)) : nrow + (blocked ? 1 : 0);
  const size_t sbase = (size_t)(b * a.hkv + g) * (a.nc + 1);
  auto pidx = [&](int j) { return (sbase + (folded || j < nrow ? j : a.nc)) * a.qr_max + qr; };
  // The output partials of the first PRE chunks do not depend on the
  // maxima: they are requested together with the chunk references, so a row
  // with up to PRE partials costs one memory round trip.
  constexpr int PRE = 16;
  float2 vp[PRE];
#pragma unroll
  for (int u = 0; u < PRE; ++u)
    vp[u] = u < ntot ? *(const float2*)(a.opart + pidx(u) * hd + lane * 2) : make_float2(0.f, 0.f);
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
    // o: lane owns dimensions 2 lane, 2 lane + 1; the first PRE chunks from
    // the registers, the rest loaded in batches of 8
    int k0 = 0;
    if (j0 == 0) {
#pragma unroll
      for (int u = 0; u < PRE; ++u) {
        if (u < n) {
          const float wu = sw[wave][u];
          o0 += vp[u].x * wu;
          o1 += vp[u].y * wu;
        }
      }
      k0 = PRE;
    }
    for (; k0 < n; k0 += 8) {
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
  const size_t oo = a.out_kb > 0 ? frag_off(r, h * hd + lane * 2, a.out_kb) : ob;
  *(uint32_t*)((uint16_t*)a.out + oo) = y;
  if (a.tap && r < a.tap_rows) *(uint32_t*)((uint16_t*)a.tap + ob) = y;
  if (a.tap32 && r < a.tap32_rows) *(float2*)(a.tap32 + ob) = make_float2(o0 * inv, o1 * inv);
}

void launch_attention_bf16(const AttnArgs& a0, hipStream_t s) {
  AttnArgs a = a0;
  const int B = a.P.B;
  const int T = a.fixed_ctx >= 0 ? a.P.Kx : a.P.tokens_per_seq();
  const int QR = T * (a.hq / a.hkv);
  // two query tiles per wave halve the K/V fragment reads per score; one
  // tile per wave gives a latency-bound launch (fewer workgroups than two
  // per compute unit) twice the workgroups with half the work each
  const int act = a.active_chunks > 0 && a.active_chunks < a.nc ? a.active_chunks : a.nc;
  if (a.tpw != 1 && a.tpw != 2) a.tpw = (long)B * a.hkv * act * attn_row_groups(QR, 2) < 512 ? 1 : 2;
  const int nrg = attn_row_groups(QR, a.tpw);
  // one row group: every key tile is read by one workgroup, so the tiles are
  // streamed past L2 (measured at 8 x 32768: verify attention 10.08 -> 9.53 ms
  // per step); with several row groups the later ones re-read the keys from
  // L2 and the default policy keeps them (the draft pass took 11.5 -> 14.5 ms
  // with non-temporal loads)
  const bool stream = nrg == 1;
  const dim3 g1((a.nc + 1) * a.hkv * B * nrg), g2(a.nc * a.hkv * B * nrg);
  if (a.tpw == 1)
    hipLaunchKernelGGL(stream ? k_attn_bf16_t1_stream : k_attn_bf16_t1, g1, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(stream ? k_attn_bf16_t2_stream : k_attn_bf16_t2, g2, dim3(256), 0, s, a);
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
