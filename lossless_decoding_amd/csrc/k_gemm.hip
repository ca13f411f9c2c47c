// Projection / FFN / LM-head GEMMs: Y[r][n] = sum_k X[r][k] W[n][k], with
// the small per-row operations of the layer fused into prologue/epilogue.
//
// bf16 path (MFMA v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//  * Operands: the packed weight is the A operand (16 output features x 32
//    k per 1 KB fragment, one coalesced wave load); the activations are the
//    B operand, staged into LDS in fragment order.
//  * Arithmetic: K is cut into 8 equal slices.  Each slice is a chain of
//    MFMAs in increasing k starting from zero; the 8 slice sums are added in
//    slice order, ((s0+s1)+s2)+...+s7.  Nothing in this order depends on the
//    number of rows, how the work is split or which rows share a launch, so
//    a row's output is identical whether computed alone (plain decoding), as
//    the anchor of a draft block or as one of K verify rows.
//  * Work split: a wave owns one 16-column tile; a workgroup of WV waves
//    owns WV*16 columns and up to max(64, 16*MT) rows (MT = 8 for passes
//    of more than 128 rows, which halves the weight re-reads).  Launches
//    with fewer than 128 (column group, row group) workgroups give every K
//    slice its own workgroup and the last workgroup of a column group adds
//    the 8 partials; the others keep all slices in one workgroup.
//  * Streaming: every wave keeps D weight fragments in flight in a register
//    ring.  Activations are staged 512 k at a time (256 at MT 8); the next stage is loaded
//    into registers one stage ahead, so waiting for it never waits for weight
//    loads issued after it (memory counters complete in order).
//  * Input: bf16 rows (RMSNorm outputs, attention output, SwiGLU product).
//  * Epilogues: QK-norm + RoPE + KV placement (QKV projection; a column
//    group is one head), SwiGLU (gate/up), per-row
//    argmax with lowest-index ties (LM head; the grid's last workgroup
//    turns the partials into tokens).  Split O and down projections write
//    their 8 slice partials and the next kernel adds them to the residual;
//    a split QKV projection writes them too and a finish kernel adds them
//    and runs its epilogue.
//
// fp32 path: one thread per output with a sequential k loop (check models).
#include "internal.h"

#include <hip/hip_ext.h>

// A GEMM launch that profiling asked to time: the dispatch itself records
// the event pair at the kernel's start and end (no gap from separate event
// records).  One pending pair per host thread, taken by the next GEMM
// kernel launched from that thread.
static thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

void gemm_time_next_launch(hipEvent_t start, hipEvent_t stop) {
  t_ev_start = start;
  t_ev_stop = stop;
}

bool gemm_time_pending() { return t_ev_start != nullptr; }

template <typename K>
static void gemm_launch(K kernel, dim3 grid, dim3 block, hipStream_t s, const GemmArgs& a) {
  if (t_ev_start) {
    hipEvent_t e0 = t_ev_start, e1 = t_ev_stop;
    t_ev_start = t_ev_stop = nullptr;
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, a);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, s, a);
  }
}


template <int N> struct IntC { static constexpr int value = N; };

#define NSL 8                 // K slices
#define SKB 16                // k-blocks of 32 per activation stage
#define BUF_FLAGS 0x00020000  // buffer descriptor word 3: 32-bit data format
#define BUF_NT 2              // cache policy: nontemporal (streamed once)
#define OOR 0x40000000        // buffer offset past every descriptor's range
#define BUF_SC1 16            // cache policy: device scope (data of other workgroups)

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

// largest divisor of n that is <= cap (at least 1)
constexpr int largest_divisor_le(int n, int cap) {
  int d = cap < n ? cap : n;
  while (d > 1 && n % d != 0) --d;
  return d < 1 ? 1 : d;
}

// QK-norm + RoPE + placement of one row's 128 outputs of column group ng
// (one head: q heads, then k heads, then v heads); lane holds columns lane
// and lane + 64.  Q goes to q_out; the K/V of mask rows to the block
// scratch, of every other row to its cache slot.
__device__ __forceinline__ void qkv_row(const GemmArgs& a, int ng, int prow, float x1, float x2,
                                        int lane) {
  const PassInfo& P = a.P;
  const int hd = 128, half = 64;
  const bool isq = ng < a.hq, isk = !isq && ng < a.hq + a.hkv;
  const int head = isq ? ng : (isk ? ng - a.hq : ng - a.hq - a.hkv);
  const RowInfo ri = row_info(P, prow);
  if (ri.pad || ri.pos >= a.cap) return;
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

// The LM head's last workgroup: each row's token from its per-column-group
// (value, index) partials amax[row][ngroups] (larger value, then lower
// index), written where the pass keeps it.  Rows row0 .. row0 + Mr - 1,
// one wave per row at a time.
__device__ __forceinline__ void amax_finish(const GemmArgs& a, int ngroups, int Mr, int row0,
                                            int wave, int nwaves, int lane) {
  for (int r = wave; r < Mr; r += nwaves) {
    const int prow = row0 + r;
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
}

// CT: 16-column tiles per wave.  With CT = 2 every activation fragment read
// from LDS feeds two MFMAs (tall row tiles, unsplit launches only).
template <int MT, int EP, int WV, bool SPLIT, int CT>
__global__ __launch_bounds__(WV * 64, (SPLIT && MT <= 2) ? 4 : 2) void k_gemm_bf16(GemmArgs a) {
  static_assert(CT == 1 || !SPLIT || EP == EP_RESID,
                "two column tiles per wave: unsplit, or split with partials only");
  constexpr int COLS = WV * 16 * CT;
  constexpr int RPW = MT * 16 > 64 ? MT * 16 : 64;     // rows per workgroup
  // k-blocks per activation stage: 16, or fewer for tall tiles (LDS stays
  // at 32-64 KB, the weight ring short); a divisor of the 16 k-blocks of a
  // slice
  // Tall row tiles (MT >= 8) stage activations straight from memory into
  // two LDS stages (no registers, no LDS writes, one barrier per stage) and
  // keep the weight ring 8 k-blocks deep (2 or 4 stages); shorter tiles go
  // through registers into one stage, the ring one stage deep.
  constexpr bool DL = MT >= 8;
  constexpr int SK = DL ? (MT >= 12 ? SKB / 8 : SKB / 4) : (MT <= 4 ? SKB : (CT == 1 ? SKB / 2 : SKB / 4));
  constexpr int NFR = MT * SK;                // activation fragments per stage
  constexpr int NF = (NFR + WV - 1) / WV;     // ... per wave
  constexpr int NSTG = DL ? 2 : 1;            // LDS activation stages
  constexpr int RING = DL ? SKB / 2 : SK;     // weight ring depth (k-blocks)
  constexpr int NU = RING / SK;               // stages per ring turn
  static_assert(RING % SK == 0 && (!DL || NU == 2 || NU == 4), "ring turns hold 2 or 4 stages");
  // LDS: the activation stages in fragment order [mt][k-block][lane][8]; in
  // the epilogue they hold fp32 output tiles (16 x COLS each), MTE at a time
  constexpr int MTE = largest_divisor_le(MT, (NSTG * MT * SK * 32 * 2) / (COLS * 4));
  static_assert(MTE >= 1 && MT % MTE == 0, "epilogue row chunks must tile MT");
  __shared__ __attribute__((aligned(16))) uint16_t sX[NSTG * MT * 16 * SK * 32];
  __shared__ float sRed[WV * RPW];
  __shared__ int sIdx[WV * RPW];
  __shared__ int sLast;

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KB = a.K >> 5;                    // k-blocks of 32
  const int KSB = KB / NSL;                   // k-blocks per slice
  const int ngroups = a.N / COLS;
  int ng, s_first, by;
  if (!SPLIT) {
    s_first = 0;
    if (a.flat) {
      // 1-D grid: the row blocks of one column group are consecutive
      // workgroups of one XCD (workgroup id mod 8), so its weights come from
      // memory once and from that XCD's L2 for the other row blocks
      const int id = blockIdx.x, j = id >> 3;
      by = j % a.gyt;
      ng = (j / a.gyt) * 8 + (id & 7);
    } else {
      ng = blockIdx.x; by = blockIdx.y;
    }
  } else if ((ngroups & 7) == 0) {            // keep a column group's slices on one XCD
    const int id = blockIdx.x;
    s_first = (id >> 3) & 7;
    ng = ((id >> 6) << 3) | (id & 7);
    by = blockIdx.y;
  } else {
    s_first = blockIdx.x % NSL;
    ng = blockIdx.x / NSL;
    by = blockIdx.y;
  }
  // row blocks [0, gy0) belong to segment 0, the rest to segment 1 (its own
  // weights and rows: the draft pass runs the mask rows' diffusion
  // projection and the anchor rows' frozen one in one launch)
  const bool seg1 = by >= a.gy0;
  const u32x4_t* const Wt = seg1 ? a.W2 : a.W;
  const int Mr = seg1 ? a.M2 : a.M;
  const int row0 = seg1 ? a.row02 : a.row0;
  const int m0 = (seg1 ? by - a.gy0 : by) * RPW;    // first row of this workgroup
  const int kb_lo = SPLIT ? s_first * KSB : 0;
  const int nkb = SPLIT ? KSB : KB;           // k-blocks of this workgroup
  const int nbk0 = (ng * WV + wave) * CT;    // this wave's first 16-column tile
  __amdgpu_buffer_rsrc_t rW[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c)
    rW[c] = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Wt + ((size_t)(nbk0 + c) * KB + kb_lo) * 64), (short)0, nkb * 1024, BUF_FLAGS);

  // stage st: k-blocks [st*SK, st*SK + SK) of this workgroup's range; the
  // lane of fragment (mt, j) holds row mt*16 + lr, k = 32 j + 8 lq .. + 7.
  // Activations and weights are read with buffer loads whose descriptors
  // cover exactly the valid rows / this wave's k-range: out-of-range loads
  // return zero without touching memory, so every load is issued
  // unconditionally, the number of loads between a ring load and its use
  // never depends on the data, and the memory-counter waits stay exact.
  const int vrows = Mr - m0 < RPW ? Mr - m0 : RPW;         // valid rows of this workgroup
  // activations in fragment order: the row tiles of this workgroup from
  // tile (row0 + m0) / 16, KB 1 KB fragments each; tiles past the valid rows
  // read as zero (rows past them inside the last tile are never stored)
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.X + (size_t)((row0 + m0) >> 4) * KB * 512), (short)0, ((vrows + 15) >> 4) * KB * 1024,
      BUF_FLAGS);
  const int a_vo = lane * 16;                                  // lane part of the offset
  u32x4_t sr[NF];
  auto load_stage = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int fr = (wave + f * WV) % NFR;
      const int mt = fr / SK, kbl = st * SK + fr % SK;
      // k-blocks past this workgroup's range are pushed out of the
      // descriptor (range checks apply to the VGPR offset)
      const int so = kbl < nkb ? (mt * KB + kb_lo + kbl) * 1024 : OOR;
      sr[f] = __builtin_amdgcn_raw_buffer_load_b128(rA, a_vo + so, 0, 0);
    }
  };
  auto write_stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int fr = wave + f * WV;
      if (fr < NFR) *(u32x4_t*)(sX + ((size_t)fr * 64 + lane) * 8) = sr[f];
    }
  };
  // direct form: fragment fr of stage st goes to LDS stage (st & 1) in lane
  // order (a buffer load with an LDS destination writes lane l's 16 bytes at
  // the stage's base + 16 l); k-blocks past the range read as zero
  auto issue_stage = [&](int st) __attribute__((always_inline)) {
    uint16_t* dst = sX + (size_t)(st & 1) * (MT * 16 * SK * 32);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int fr = wave + f * WV;
      if (fr < NFR) {
        const int mt = fr / SK, kbl = st * SK + fr % SK;
        const int so = kbl < nkb ? (mt * KB + kb_lo + kbl) * 1024 : OOR;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rA, (__attribute__((address_space(3))) void*)(dst + (size_t)fr * 512), 16, a_vo + so, 0, 0, 0);
      }
    }
  };
  const int nst0 = (nkb + SK - 1) / SK;      // activation stages
  const int nst = DL ? (nst0 + NU - 1) / NU * NU : nst0;   // direct form: whole ring turns (extra stages add zeros)
  if (DL) issue_stage(0);
  else load_stage(0);
  // weight ring: slot j holds k-block j (mod RING) ahead of use; loads past
  // this wave's k-range fall outside the descriptor (zero, no memory access)
  u32x4_t w[CT][RING];
#pragma unroll
  for (int i = 0; i < RING; ++i)
#pragma unroll
    for (int c = 0; c < CT; ++c)
      w[c][i] = __builtin_amdgcn_raw_buffer_load_b128(rW[c], lane * 16 + i * 1024, 0, BUF_NT);

  if (!DL) {
    write_stage();
    __syncthreads();
  }

  floatx4_t cur[CT][MT], tot[CT][MT];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      cur[c][mt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      tot[c][mt] = cur[c][mt];
    }
  // Per stage: switch the LDS stage, prefetch the next one, then SK MFMA
  // steps, each refilling its ring slot with the k-block one stage ahead.
  // The loads are the same on every path.  Past the end of a partial last
  // stage both operands are zero, so the extra MFMAs add exact zeros.
  // SK MFMA steps of stage st from LDS stage `buf`, each refilling its ring
  // slot (sub-stage u of the ring) with the k-block RING ahead
  auto compute_stage = [&](int st, const uint16_t* buf, auto uc) __attribute__((always_inline)) {
    constexpr int U = decltype(uc)::value;
#pragma unroll
    for (int i = 0; i < SK; ++i) {
      const int kk = st * SK + i;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4_t xv = *(const u32x4_t*)(buf + ((size_t)(mt * SK + i) * 64 + lane) * 8);
#pragma unroll
        for (int c = 0; c < CT; ++c)
          cur[c][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w[c][U * SK + i]),
                                                               as_bf16x8(xv), cur[c][mt], 0, 0, 0);
      }
#pragma unroll
      for (int c = 0; c < CT; ++c)
        w[c][U * SK + i] =
            __builtin_amdgcn_raw_buffer_load_b128(rW[c], lane * 16 + (kk + RING) * 1024, 0, BUF_NT);
      if (!SPLIT && kk < nkb && (kk + 1) % KSB == 0) {   // slice done: add in slice order
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            tot[c][mt] = kk + 1 == KSB ? cur[c][mt] : add4(tot[c][mt], cur[c][mt]);
            cur[c][mt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
          }
      }
    }
  };
  if constexpr (DL) {
    // Stage st: wait for this wave's loads of stage st (only the weight
    // loads issued after them may still be in flight: RING loads before the
    // first stage, SK per stage after) and for its LDS reads of the
    // previous stage; the barrier then makes every wave's share visible and
    // frees the other LDS stage, which takes stage st + 1.
    constexpr int W0 = RING * CT, W1 = SK * CT;
    static_assert(W0 < 64 && W1 < 64, "vmcnt range");
    constexpr int E0 = (W0 & 15) | ((W0 >> 4) << 14) | (7 << 4);   // vmcnt(W0) lgkmcnt(0)
    constexpr int E1 = (W1 & 15) | ((W1 >> 4) << 14) | (7 << 4);   // vmcnt(W1) lgkmcnt(0)
    auto sync_stage = [&](bool first) __attribute__((always_inline)) {
      if (first) __builtin_amdgcn_s_waitcnt(E0);
      else __builtin_amdgcn_s_waitcnt(E1);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    for (int st0 = 0; st0 < nst; st0 += NU) {
      // one ring turn: stage st0 + u reads LDS stage u & 1 and ring slots
      // [u SK, u SK + SK)
      auto one = [&](auto uc) __attribute__((always_inline)) {
        constexpr int U = decltype(uc)::value;
        const int st = st0 + U;
        sync_stage(st == 0);
        if (st + 1 < nst) issue_stage(st + 1);
        compute_stage(st, sX + (U & 1) * (MT * 16 * SK * 32), uc);
      };
      one(IntC<0>{});
      one(IntC<1>{});
      if constexpr (NU == 4) {
        one(IntC<2>{});
        one(IntC<3>{});
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
  } else {
    for (int st = 0; st < nst; ++st) {
      if (st > 0) {
        __syncthreads();                 // every wave is done with the previous stage
        write_stage();
        __syncthreads();
      }
      load_stage(st + 1);
      compute_stage(st, sX, IntC<0>{});
    }
  }
  if (!SPLIT) {
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) cur[c][mt] = tot[c][mt];
  }
  floatx4_t (&cs)[MT] = cur[0];               // the only tile when CT = 1

  // ---- split-K residual and QKV GEMMs: the slice partial goes to
  // [slice][row][N]; the kernel that follows (residual + RMSNorm, or the QKV
  // finish) adds the 8 partials in slice order, so no workgroup waits for
  // another here.
  if (SPLIT && (EP == EP_RESID || EP == EP_QKV)) {
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = m0 + mt * 16 + lr;
        if (r < Mr)
          *(floatx4_t*)(a.rpart + (size_t)s_first * a.rps + (size_t)(row0 + r) * a.N + (nbk0 + c) * 16 +
                        lq * 4) = cur[c][mt];
      }
    return;
  }
  // ---- split-K: write the slice partial; the last slice workgroup adds all 8.
  // Partials and counters use device-scope (coherent) stores and loads; an
  // explicit wait for the stores plus the barrier orders them before the
  // counter increment, so no L2 writeback is needed.
  if (SPLIT) {
    // partial layout [slice][m-group][col group][mt][wave][lane][4]: one
    // 16-byte device-scope store / load per lane and row tile (a wave moves
    // 1 KB contiguous)
    const size_t pstride = (size_t)a.gyt * ngroups * MT * WV * 256;
    float* pbase = a.part + ((size_t)by * ngroups + ng) * MT * WV * 256;
    const __amdgpu_buffer_rsrc_t rPt =
        __builtin_amdgcn_make_buffer_rsrc((void*)pbase, (short)0, 0x7fffffff, BUF_FLAGS);
    auto poff = [&](int s, int mt) {
      return (int)((s * pstride + ((size_t)mt * WV + wave) * 256) * 4) + lane * 16;
    };
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, cs[mt]), rPt,
                                             poff(s_first, mt), 0, BUF_SC1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      unsigned* cp = a.cnt + by * ngroups + ng;
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
        if (s == s_first) p[s] = cs[mt];
        else p[s] = __builtin_bit_cast(floatx4_t,
                                       __builtin_amdgcn_raw_buffer_load_b128(rPt, poff(s, mt), 0, BUF_SC1));
      }
      floatx4_t t = p[0];
#pragma unroll
      for (int s = 1; s < NSL; ++s) t = add4(t, p[s]);
      cs[mt] = t;
    }
  }

  // ============================ epilogues
  // lane (lr, lq) of wave w holds rows m0 + mt*16 + lr, columns (nbk0 + c)*16 + lq*4 + i
  float* tile = (float*)sX;                  // [MT*16][COLS] fp32 scratch
  __syncthreads();
  if (EP == EP_RESID) {
    // h += y
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = m0 + mt * 16 + lr;
        if (r < Mr) {
          float* yp = a.y + (size_t)(row0 + r) * a.ldy + (nbk0 + c) * 16 + lq * 4;
          float4 o = *(float4*)yp;
          o.x += cur[c][mt][0]; o.y += cur[c][mt][1]; o.z += cur[c][mt][2]; o.w += cur[c][mt][3];
          *(float4*)yp = o;
        }
      }
    return;
  }
  if (EP == EP_SWIGLU && CT == 2) {
    // gate (even tile) and up (odd tile) of one 16-column act block are this
    // wave's two tiles
    const int j = (nbk0 >> 1) * 16 + lq * 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = m0 + mt * 16 + lr;
      if (r >= Mr) continue;
      uint16_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = f2bf(silu_f(cur[0][mt][i]) * cur[CT - 1][mt][i]);
      uint2 pk;
      __builtin_memcpy(&pk, o, 8);
      *(uint2*)(a.act + frag_off(row0 + r, j, a.ldact >> 5)) = pk;
    }
    return;
  }
  if (EP == EP_SWIGLU) {
    // odd waves hold the up block of the even wave before them; MTE row
    // tiles at a time through the LDS tile
#pragma unroll
    for (int mc = 0; mc < MT; mc += MTE) {
      if (mc > 0) __syncthreads();       // the previous chunk's tile is read
      if (wave & 1) {
#pragma unroll
        for (int e = 0; e < MTE; ++e)
          *(floatx4_t*)(tile + ((e * 16 + lr) * COLS) + (wave >> 1) * 16 + lq * 4) = cs[mc + e];
      }
      __syncthreads();
      if (!(wave & 1)) {
#pragma unroll
        for (int e = 0; e < MTE; ++e) {
          const int mt = mc + e;
          int r = m0 + mt * 16 + lr;
          if (r >= Mr) continue;
          floatx4_t u = *(const floatx4_t*)(tile + ((e * 16 + lr) * COLS) + (wave >> 1) * 16 + lq * 4);
          int j = (ng * (WV / 2) + (wave >> 1)) * 16 + lq * 4;
          uint16_t o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = f2bf(silu_f(cs[mt][i]) * u[i]);
          uint2 pk;
          __builtin_memcpy(&pk, o, 8);
          *(uint2*)(a.act + frag_off(row0 + r, j, a.ldact >> 5)) = pk;
        }
      }
    }
    return;
  }
  if (EP == EP_ARGMAX) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      int r = m0 + mt * 16 + lr;
      float bv = cur[0][mt][0];
      int bi = nbk0 * 16 + lq * 4;
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (c > 0 || i > 0) amax_comb(bv, bi, cur[c][mt][i], (nbk0 + c) * 16 + lq * 4 + i);
      if (a.logits && r < Mr) {
#pragma unroll
        for (int c = 0; c < CT; ++c)
          *(floatx4_t*)(a.logits + (size_t)(row0 + r) * a.ldl + (nbk0 + c) * 16 + lq * 4) = cur[c][mt];
      }
      float v2 = __shfl_xor(bv, 16, 64); int i2 = __shfl_xor(bi, 16, 64);
      amax_comb(bv, bi, v2, i2);
      v2 = __shfl_xor(bv, 32, 64); i2 = __shfl_xor(bi, 32, 64);
      amax_comb(bv, bi, v2, i2);
      if (lq == 0) { sRed[wave * RPW + mt * 16 + lr] = bv; sIdx[wave * RPW + mt * 16 + lr] = bi; }
    }
    __syncthreads();
    if (tid < MT * 16 && m0 + tid < Mr) {
      float bv = sRed[tid];
      int bi = sIdx[tid];
      for (int w = 1; w < WV; ++w) amax_comb(bv, bi, sRed[w * RPW + tid], sIdx[w * RPW + tid]);
      float2* ap = a.amax + (size_t)(row0 + m0 + tid) * ngroups + ng;
      st_agent(&ap->x, bv);
      st_agent(&ap->y, __int_as_float(bi));
    }
    // the grid's last surviving workgroup turns the per-group partials into tokens
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      unsigned* cp = a.cnt + a.gyt * ngroups;
      unsigned old = __hip_atomic_fetch_add(cp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      unsigned total = (unsigned)ngroups * a.gyt;   // one workgroup per (column group, row block)
      sLast = old == total - 1;
      if (old == total - 1) __hip_atomic_store(cp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!sLast) return;
    amax_finish(a, ngroups, Mr, row0, wave, WV, lane);
    return;
  }
  if (EP == EP_QKV) {
    // column group ng is one head: q heads, then k heads, then v heads; MTE
    // row tiles at a time through the LDS tile
#pragma unroll
    for (int mc = 0; mc < MT; mc += MTE) {
      if (mc > 0) __syncthreads();       // the previous chunk's rows are done
#pragma unroll
      for (int e = 0; e < MTE; ++e)
#pragma unroll
        for (int c = 0; c < CT; ++c)
          *(floatx4_t*)(tile + ((e * 16 + lr) * COLS) + (wave * CT + c) * 16 + lq * 4) = cur[c][mc + e];
      __syncthreads();
      for (int rl = wave; rl < MTE * 16; rl += WV) {
        const int r = m0 + mc * 16 + rl;
        if (r >= Mr) break;
        qkv_row(a, ng, row0 + r, tile[rl * COLS + lane], tile[rl * COLS + lane + 64], lane);
      }
    }
    return;
  }
}

// Split QKV projection, second half: one wave per (row, head) adds the 8
// slice partials in slice order and runs the QK-norm / RoPE / placement
// epilogue.  Rows [0, M) are segment 0 (from row0), [M, M + M2) segment 1.
// NS = 1: an unsplit launch stored its slice-ordered sums in slice 0.
template <int NS>
__global__ __launch_bounds__(64) void k_qkv_finish_bf16(GemmArgs a) {
  const int r = blockIdx.x, ng = blockIdx.y, lane = threadIdx.x;
  const int prow = r < a.M ? a.row0 + r : a.row02 + (r - a.M);
  const float* p = a.rpart + (size_t)prow * a.N + ng * 128 + lane;
  float x1 = p[0], x2 = p[64];
#pragma unroll
  for (int sl = 1; sl < NS; ++sl) {
    x1 += p[(size_t)sl * a.rps];
    x2 += p[(size_t)sl * a.rps + 64];
  }
  qkv_row(a, ng, prow, x1, x2, lane);
}

// ------------------------------------------------------------ row-split form
// Launches of 256 rows and more (draft / verify passes of several
// sequences, prefill passes).  A workgroup of four waves owns C column
// tiles and one row block of up to 3 TRW + TRW0 row tiles (16 rows each),
// which the waves split: waves 1-3 take TRW tiles each, wave 0 the rest
// (at most TRW0) and loads the workgroup's weights.  Each weight fragment
// is loaded once per workgroup, straight from memory into LDS (buffer loads
// with an LDS destination, TNS stages of TS k-blocks in flight), and read
// from LDS by all four waves.  Each wave loads its own activation fragments
// into a register ring TDX k-blocks deep.  Memory counters complete in issue
// order, so a wave that waits for an activation load also waits for every
// older load; keeping the weight loads in wave 0 lets the other waves wait
// for their activations only.  Per k-block a wave reads C weight fragments
// from LDS and issues (tiles) x C MFMAs.
//  * The arithmetic of every output is the slice order of the kernel above
//    (same MFMA, same operands, same slice sums), so the two forms give
//    identical bits for a row.
//  * Two segments (mask rows with one weight set, anchor rows with another)
//    may share a row block: the workgroup then stages both weight sets.
//  * Split launches (O, down, QKV) give each K slice its own workgroup and
//    write the slice partials for the next kernel; unsplit launches run the
//    SwiGLU or argmax epilogue, or (O, down and QKV in prefill passes, whose
//    row blocks alone fill the chip) add their sums to the residual in place
//    or store them for the QKV finish kernel.
#define TRW 5    // row tiles of waves 1-3
#define TRW0 2   // row tiles of wave 0 (the weight loader)

template <int C, int EP, bool SPLIT, bool TWO>
__global__ __launch_bounds__(256, 1) void k_gemm_rows(GemmArgs a) {
  static_assert(SPLIT ? (EP == EP_RESID || EP == EP_QKV)
                      : (EP == EP_SWIGLU || EP == EP_ARGMAX || EP == EP_RESID || EP == EP_QKV),
                "split launches write partials; unsplit ones run SwiGLU, argmax, the residual add or "
                "store QKV sums");
  static_assert(!TWO || SPLIT, "two weight sets: split launches only");
  static_assert(EP != EP_SWIGLU || C % 2 == 0, "SwiGLU pairs gate and up tiles");
  constexpr int NW = TWO ? 2 * C : C;           // weight fragments per k-block
  // k-blocks per weight stage: one for the widest workgroups, so that wave
  // 0's prologue wait stays within the memory counter's range
  constexpr int TS = (NW > 12 || C >= 12) ? 1 : 2;
  constexpr int LPS = NW * TS;                  // weight loads (1 KB) per stage, all by wave 0
  constexpr int TNS = TWO ? 4 : 5;              // weight stages in LDS
  constexpr int TDX = TWO ? 4 : 5;              // activation ring depth (k-blocks)
  static_assert((TNS * TS) % TDX == 0, "ring slots stay compile-time over a ring turn");
  constexpr int SU = LPS * 512;                 // one stage (uint16 elements)
  static_assert(TNS * SU * 2 <= 160 * 1024, "LDS");
  // one array per stage, so the compiler sees that loads into one stage and
  // reads of another do not alias (no wait for the loads in flight)
  __shared__ __attribute__((aligned(16))) uint16_t sW0[SU];
  __shared__ __attribute__((aligned(16))) uint16_t sW1[SU];
  __shared__ __attribute__((aligned(16))) uint16_t sW2[SU];
  __shared__ __attribute__((aligned(16))) uint16_t sW3[SU];
  __shared__ __attribute__((aligned(16))) uint16_t sW4[TNS > 4 ? SU : 8];
  auto stage_buf = [&](auto uc) __attribute__((always_inline)) -> uint16_t* {
    constexpr int S = decltype(uc)::value % TNS;
    if constexpr (S == 0) return sW0;
    else if constexpr (S == 1) return sW1;
    else if constexpr (S == 2) return sW2;
    else if constexpr (S == 3) return sW3;
    else return sW4;
  };

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KB = a.K / 32;
  const int KSB = KB / NSL;
  const int nsl = SPLIT ? NSL : 1;
  // 1-D grid; the row blocks of one (column group, slice) are consecutive
  // workgroups of one XCD (workgroup id mod 8), so a weight fragment comes
  // from memory once and from that XCD's L2 for the other row blocks
  const int id = blockIdx.x, j8 = id >> 3;
  const int gq = j8 / a.tnrb, rb = j8 - gq * a.tnrb;
  const int grp = gq * 8 + (id & 7);
  if (grp >= a.tng * nsl) return;
  const int ng = SPLIT ? grp / NSL : grp;
  const int sl = SPLIT ? grp - ng * NSL : 0;
  const int kb_lo = sl * KSB;
  const int nkb = SPLIT ? KSB : KB;
  const int ntiles = a.N / 16;                  // column tiles of the matrix
  const int ct0 = ng * C;                       // first column tile of the workgroup
  const int nct = min(C, ntiles - ct0);         // its valid column tiles

  // row tiles: segment 0 (M rows from row0) then segment 1 (M2 rows from
  // row02); this block's nb tiles: wave 0 the first n0, then TRW per wave
  const int T0 = (a.M + 15) >> 4;
  const int T = T0 + ((a.M2 + 15) >> 4);
  const int tb0 = rb * a.ttb;
  const int nb = min(a.ttb, T - tb0);
  const int n0 = max(0, nb - 3 * TRW);          // <= TRW0 (launcher)
  const int my_lo = wave == 0 ? 0 : n0 + (wave - 1) * TRW;
  const int ntw = wave == 0 ? n0 : max(0, min(TRW, nb - my_lo));   // uniform
  __amdgpu_buffer_rsrc_t rX[TRW];
  int rowb[TRW], vrow[TRW];
  bool s1[TRW];
#pragma unroll
  for (int jj = 0; jj < TRW; ++jj) {
    const int gt = tb0 + my_lo + jj;
    s1[jj] = TWO && gt >= T0;
    const int rbase = s1[jj] ? a.row02 + (gt - T0) * 16 : a.row0 + gt * 16;
    int v = s1[jj] ? a.M2 - (gt - T0) * 16 : a.M - gt * 16;
    v = jj < ntw ? (v < 16 ? v : 16) : 0;
    rowb[jj] = rbase; vrow[jj] = v;
    // fragment order: tile rbase / 16, KB fragments of 1 KB (rows past the
    // valid ones inside the tile are never stored)
    rX[jj] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.X + (size_t)(v > 0 ? rbase >> 4 : 0) * KB * 512),
                                               (short)0, v > 0 ? KB * 1024 : 0, BUF_FLAGS);
  }
  const int x_vo = lane * 16;
  // weights: the workgroup's C column tiles are contiguous ([tile][k-block][1 KB])
  const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.W + (size_t)ct0 * KB * 64), (short)0, nct * KB * 1024, BUF_FLAGS);
  __amdgpu_buffer_rsrc_t rW2 = rW;
  if (TWO)
    rW2 = __builtin_amdgcn_make_buffer_rsrc((void*)(a.W2 + (size_t)ct0 * KB * 64), (short)0,
                                            nct * KB * 1024, BUF_FLAGS);

  // stage st (wave 0): the NW fragments of k-blocks st*TS .. st*TS+TS-1
  // into LDS ([k-block][fragment] of 1 KB, lane order); k-blocks past the
  // range read as zero
  auto issue_w = [&](uint16_t* buf, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TS; ++i) {
      const int kk = st * TS + i;
      const int ko = kk < nkb ? (kb_lo + kk) * 1024 + lane * 16 : OOR;
#pragma unroll
      for (int f = 0; f < NW; ++f) {
        const bool second = TWO && f >= C;
        const int c = second ? f - C : f;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            second ? rW2 : rW, (__attribute__((address_space(3))) void*)(buf + (i * NW + f) * 512), 16,
            ko == OOR ? OOR : c * KB * 1024 + ko, 0, 0, BUF_NT);
      }
    }
  };
  u32x4_t xr[TDX][TRW];
  floatx4_t cur[TRW][C];
  floatx4_t tot[SPLIT ? 1 : TRW][SPLIT ? 1 : C];
#pragma unroll
  for (int jj = 0; jj < TRW; ++jj)
#pragma unroll
    for (int c = 0; c < C; ++c) cur[jj][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (!SPLIT) {
#pragma unroll
    for (int jj = 0; jj < TRW; ++jj)
#pragma unroll
      for (int c = 0; c < C; ++c) tot[jj][c] = cur[jj][c];
  }
  const int nst = (nkb + TS - 1) / TS;
  int next_end = KSB;                           // k-block count at the end of the current slice

  // The main loop for a wave of R row tiles (wave 0: R = TRW0, the loader).
  auto main_loop = [&](auto rc) __attribute__((always_inline)) {
    constexpr int R = decltype(rc)::value;
    constexpr bool LD = R == TRW0;
    auto issue_x = [&](int kk, u32x4_t (&dst)[TRW]) __attribute__((always_inline)) {
      const int so = kk < nkb ? (kb_lo + kk) * 1024 : OOR;
#pragma unroll
      for (int jj = 0; jj < R; ++jj) dst[jj] = __builtin_amdgcn_raw_buffer_load_b128(rX[jj], x_vo + so, 0, 0);
    };
    if constexpr (LD) {
#pragma unroll
      for (int p = 0; p < TNS - 1; ++p) {
        if (p == 0) issue_w(stage_buf(IntC<0>{}), 0);
        else if (p == 1) issue_w(stage_buf(IntC<1>{}), 1);
        else if (p == 2) issue_w(stage_buf(IntC<2>{}), 2);
        else issue_w(stage_buf(IntC<3>{}), 3);
      }
    }
#pragma unroll
    for (int d = 0; d < TDX; ++d) issue_x(d, xr[d]);
    // wave 0's waits for stage st's weights: the loads issued after them are
    // the later prologue stages and the prologue activations (first TNS-1
    // stages, fewer), or TNS-1 stages of activations and TNS-2 of weights
    constexpr int N0 = (TNS - 2) * LPS + TDX * R;
    constexpr int NA0 = (TNS - 1) * TS * R + (TNS - 2) * LPS;
    constexpr int NA = NA0 < 63 ? NA0 : 63;
    static_assert(!LD || N0 <= 63, "prologue wait within the counter's range");
    constexpr int E0 = (N0 & 15) | ((N0 >> 4) << 14) | (7 << 4);   // vmcnt(N0) lgkmcnt(0)
    constexpr int EA = (NA & 15) | ((NA >> 4) << 14) | (7 << 4);   // vmcnt(NA) lgkmcnt(0)
    constexpr int EL = 15 | (3 << 14) | (7 << 4);                  // lgkmcnt(0)

    for (int st0 = 0; st0 < nst; st0 += TNS) {
      auto one = [&](auto uc) __attribute__((always_inline)) {
        constexpr int U = decltype(uc)::value;
        const int st = st0 + U;
        // stage st's weights are in LDS and every wave's reads of stage
        // st-1 are done: wave 0 waits for its loads, every wave for its
        // LDS reads, then the barrier; stage st-1's buffer takes stage
        // st + TNS - 1
        if constexpr (LD) {
          if (st < TNS - 1) __builtin_amdgcn_s_waitcnt(E0);
          else __builtin_amdgcn_s_waitcnt(EA);
        } else {
          __builtin_amdgcn_s_waitcnt(EL);
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if constexpr (LD) issue_w(stage_buf(IntC<U + TNS - 1>{}), st + TNS - 1);
        const uint16_t* buf = stage_buf(IntC<U>{});
#pragma unroll
        for (int i = 0; i < TS; ++i) {
          const int kk = st * TS + i;
          u32x4_t (&xv)[TRW] = xr[(U * TS + i) % TDX];
          u32x4_t wf[C], wf2[TWO ? C : 1];
#pragma unroll
          for (int c = 0; c < C; ++c) wf[c] = *(const u32x4_t*)(buf + ((i * NW + c) * 64 + lane) * 8);
          if constexpr (TWO) {
            bool any2 = false;
#pragma unroll
            for (int jj = 0; jj < R; ++jj) any2 = any2 || (jj < ntw && s1[jj]);
            if (any2) {
#pragma unroll
              for (int c = 0; c < C; ++c) wf2[c] = *(const u32x4_t*)(buf + ((i * NW + C + c) * 64 + lane) * 8);
            } else {
#pragma unroll
              for (int c = 0; c < C; ++c) wf2[c] = wf[c];
            }
          }
#pragma unroll
          for (int jj = 0; jj < R; ++jj) {
            if (jj >= ntw) break;
            if (TWO && s1[jj]) {
#pragma unroll
              for (int c = 0; c < C; ++c)
                cur[jj][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wf2[TWO ? c : 0]),
                                                                    as_bf16x8(xv[jj]), cur[jj][c], 0, 0, 0);
            } else {
#pragma unroll
              for (int c = 0; c < C; ++c)
                cur[jj][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wf[c]), as_bf16x8(xv[jj]),
                                                                    cur[jj][c], 0, 0, 0);
            }
          }
          issue_x(kk + TDX, xv);
          // slice done: add it in slice order.  tot starts at +0 and a slice
          // sum is never -0 (its chain starts at +0), so the first addition
          // gives the slice sum exactly.  (Unsplit launches have no k-blocks
          // past the range: KB is a multiple of 8.)  The empty asm keeps this
          // a branch taken 8 times, not selects at every k-block.
          if constexpr (!SPLIT) {
            if (kk + 1 == next_end) {
              asm volatile("" ::: "memory");
              next_end += KSB;
#pragma unroll
              for (int jj = 0; jj < R; ++jj)
#pragma unroll
                for (int c = 0; c < C; ++c) {
                  tot[jj][c] = add4(tot[jj][c], cur[jj][c]);
                  cur[jj][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
                }
            }
          }
        }
      };
      one(IntC<0>{});
      if (st0 + 1 < nst) one(IntC<1>{});
      if (st0 + 2 < nst) one(IntC<2>{});
      if (st0 + 3 < nst) one(IntC<3>{});
      if constexpr (TNS > 4) {
        if (st0 + 4 < nst) one(IntC<4>{});
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
  };
  if (wave == 0) main_loop(IntC<TRW0>{});
  else main_loop(IntC<TRW>{});
  if constexpr (!SPLIT) {
#pragma unroll
    for (int jj = 0; jj < TRW; ++jj)
#pragma unroll
      for (int c = 0; c < C; ++c) cur[jj][c] = tot[jj][c];
  }

  // ============================ epilogues
  // lane (lr, lq): rows rowb[jj] + lr, columns (ct0 + c)*16 + lq*4 + i
  // split launches: slice sl's partials; unsplit QKV: the slice-ordered
  // sums, as slice 0 (the finish kernel then adds nothing)
  if constexpr (SPLIT || EP == EP_QKV) {
#pragma unroll
    for (int jj = 0; jj < TRW; ++jj) {
      if (lr >= vrow[jj]) continue;
      float* pp = a.rpart + (size_t)sl * a.rps + (size_t)(rowb[jj] + lr) * a.N + ct0 * 16 + lq * 4;
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (c < nct) *(floatx4_t*)(pp + c * 16) = cur[jj][c];
    }
    return;
  }
  if constexpr (EP == EP_RESID) {
    // the residual add in place, h + (slice-ordered sum): the value the
    // residual-norm kernel forms from a split launch's partials
#pragma unroll
    for (int jj = 0; jj < TRW; ++jj) {
      if (lr >= vrow[jj]) continue;
      float* yp = a.y + (size_t)(rowb[jj] + lr) * a.ldy + ct0 * 16 + lq * 4;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        if (c >= nct) break;
        floatx4_t hv = *(const floatx4_t*)(yp + c * 16);
        hv[0] += cur[jj][c][0]; hv[1] += cur[jj][c][1];
        hv[2] += cur[jj][c][2]; hv[3] += cur[jj][c][3];
        *(floatx4_t*)(yp + c * 16) = hv;
      }
    }
    return;
  }
  if constexpr (EP == EP_SWIGLU) {
    // gate (even tile) and up (odd tile) of one 16-column act block
#pragma unroll
    for (int jj = 0; jj < TRW; ++jj) {
      if (lr >= vrow[jj]) continue;
#pragma unroll
      for (int c = 0; c < C; c += 2) {
        if (c >= nct) break;
        uint16_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = f2bf(silu_f(cur[jj][c][i]) * cur[jj][c + 1][i]);
        uint2 pk;
        __builtin_memcpy(&pk, o, 8);
        *(uint2*)(a.act + frag_off(rowb[jj] + lr, ((ct0 + c) >> 1) * 16 + lq * 4, a.ldact >> 5)) = pk;
      }
    }
    return;
  }
  if constexpr (EP == EP_ARGMAX) {
#pragma unroll
    for (int jj = 0; jj < TRW; ++jj) {
      if (jj >= ntw) break;
      float bv = cur[jj][0][0];
      int bi = ct0 * 16 + lq * 4;
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((c > 0 || i > 0) && c < nct) amax_comb(bv, bi, cur[jj][c][i], (ct0 + c) * 16 + lq * 4 + i);
      if (a.logits && lr < vrow[jj]) {
#pragma unroll
        for (int c = 0; c < C; ++c)
          if (c < nct)
            *(floatx4_t*)(a.logits + (size_t)(rowb[jj] + lr) * a.ldl + (ct0 + c) * 16 + lq * 4) = cur[jj][c];
      }
      float v2 = __shfl_xor(bv, 16, 64); int i2 = __shfl_xor(bi, 16, 64);
      amax_comb(bv, bi, v2, i2);
      v2 = __shfl_xor(bv, 32, 64); i2 = __shfl_xor(bi, 32, 64);
      amax_comb(bv, bi, v2, i2);
      if (lq == 0 && lr < vrow[jj]) {
        float2* ap = a.amax + (size_t)(rowb[jj] + lr) * a.tng + ng;
        st_agent(&ap->x, bv);
        st_agent(&ap->y, __int_as_float(bi));
      }
    }
    // k_amax_rows, launched next, turns the per-group partials into tokens
    return;
  }
}

// The row-split LM head's second half: one wave per row reduces the row's
// per-column-group (value, index) partials.
__global__ __launch_bounds__(64) void k_amax_rows(GemmArgs a) {
  amax_finish(a, a.tng, a.M, a.row0, blockIdx.x, gridDim.x, threadIdx.x);
}

template <int EP, int WV, bool SPLIT, int CT = 1>
static void dispatch_mt(int MT, dim3 grid, const GemmArgs& a, hipStream_t s) {
  const dim3 block(WV * 64);
  switch (MT) {
    case 1: gemm_launch(k_gemm_bf16<1, EP, WV, SPLIT, CT>, grid, block, s, a); break;
    case 2: gemm_launch(k_gemm_bf16<2, EP, WV, SPLIT, CT>, grid, block, s, a); break;
    case 3: gemm_launch(k_gemm_bf16<3, EP, WV, SPLIT, CT>, grid, block, s, a); break;
    case 4: gemm_launch(k_gemm_bf16<4, EP, WV, SPLIT, CT>, grid, block, s, a); break;
    case 8: gemm_launch(k_gemm_bf16<8, EP, WV, SPLIT, CT>, grid, block, s, a); break;
    case 9:   // unsplit launches only (tall-tile rule)
      if constexpr (!SPLIT) gemm_launch(k_gemm_bf16<9, EP, WV, SPLIT, CT>, grid, block, s, a);
      break;
    case 12: gemm_launch(k_gemm_bf16<12, EP, WV, SPLIT, CT>, grid, block, s, a); break;
    default: gemm_launch(k_gemm_bf16<16, EP, WV, SPLIT, CT>, grid, block, s, a); break;
  }
}

// unsplit gate/up launches of 128- or 144-row tiles: four waves of two
// column tiles (128 columns: gate and up in one wave).  Measured: faster for
// gate/up at 256-512 rows; slower for QKV and the LM head, whose grids keep
// fewer loads in flight with four waves per workgroup.  Taller tiles would
// not fit two tiles' accumulators.
template <int EP>
static void dispatch_ct2(int MT, dim3 grid, const GemmArgs& a, hipStream_t s) {
  if (MT == 9) gemm_launch(k_gemm_bf16<9, EP, 4, false, 2>, grid, dim3(256), s, a);
  else gemm_launch(k_gemm_bf16<8, EP, 4, false, 2>, grid, dim3(256), s, a);
}

int gemm_bf16_groups(int N) { return N / 128; }

// Row tiles (16 rows) per workgroup: the rows rounded up to tiles up to 64
// rows, 4 (64 rows) up to 128, 8 (128 rows) beyond.  This sets the row
// groups that decide whether K is split.
static int gemm_mt(int M, int M2) {
  const int Mx = M > M2 ? M : M2;
  return Mx > 128 ? 8 : (Mx >= 64 ? 4 : (Mx + 15) / 16);
}

// rows per workgroup of a launch (both segments) under gemm_mt
static int gemm_rows_per_wg(int M, int M2) {
  const int MT = gemm_mt(M, M2);
  return MT > 4 ? MT * 16 : 64;
}

// An unsplit single-segment launch of more than 128 rows may take taller
// row tiles (MT 12 or 16: 192 or 256 rows), which read the weights fewer
// times through the caches.  The MFMA operand reads from LDS per row do not
// change, so what decides is padding: the tile with the fewest padded rows
// (the smaller on ties) among those that keep at least 512 workgroups, then
// 144-row tiles (MT 9) if they pad fewer still (264 rows: 2 x 144).
static int gemm_mt_tall(int M, int M2, int ngroups) {
  if (M2 > 0 || M <= 128) return gemm_mt(M, M2);
  int best = 8;
  long best_rows = (long)((M + 127) / 128) * 128;
  for (int MT = 12; MT <= 16; MT += 4) {
    const int g = (M + MT * 16 - 1) / (MT * 16);
    const long rows = (long)g * MT * 16;
    if ((long)ngroups * g >= 512 && rows < best_rows) { best = MT; best_rows = rows; }
  }
  const int g9 = (M + 143) / 144;
  if ((long)ngroups * g9 >= 512 && (long)g9 * 144 < best_rows) best = 9;
  return best;
}

// 144-row tiles pad fewer rows than 128-row ones (528 rows: 576 against 640)
static bool rows144_pad_less(int M) { return (M + 143) / 144 * 144 < (M + 127) / 128 * 128; }

// Split K over workgroups only when the column groups times the row groups
// of the launch are too few to fill the chip without it: fewer than 128,
// or fewer than 256 for EP_RESID, whose split form only writes partials (no
// in-kernel fixup).  0 or the number of K slices: for EP_RESID the residual
// + RMSNorm kernel that follows must add that many slice partials.
// The row-split form (k_gemm_rows) takes launches of at least 16 row tiles
// (256 rows) with 16-column tiles in whole pairs: SwiGLU and argmax unsplit
// (one weight set); QKV and the residual GEMMs split into the 8 K slices,
// except in launches whose row blocks alone give two full rounds (prefill
// passes).  Column tiles per workgroup: 6 for SwiGLU (the Qwen3-8B gate/up
// GEMM is then one workgroup per compute unit at 272 rows), argmax and
// two-segment QKV; split, 12 for one-segment QKV and 8 for the residual
// GEMMs; unsplit, 4 for QKV and the residual GEMMs.  Row blocks of at most
// 3 * TRW + TRW0 tiles, balanced.
struct RowsPlan { int C, two, split, nrb, tb, ng, wgs; };

static bool rows_plan(int M, int M2, int N, int ep, RowsPlan& p) {
  if (M2 < 0) M2 = 0;
  const int T = (M + 15) / 16 + (M2 + 15) / 16;
  if (T < 16 || N % 32 != 0) return false;
  if ((ep == EP_SWIGLU || ep == EP_ARGMAX) && M2 > 0) return false;
  if (ep != EP_SWIGLU && ep != EP_ARGMAX && ep != EP_RESID && ep != EP_QKV) return false;
  p.two = M2 > 0;
  p.nrb = (T + 3 * TRW + TRW0 - 1) / (3 * TRW + TRW0);
  p.tb = (T + p.nrb - 1) / p.nrb;
  // QKV and the residual GEMMs split K unless their row blocks alone give
  // two full rounds of workgroups at 4 column tiles (prefill passes), where
  // the slice partials would only add memory traffic (unsplit QKV still
  // leaves its sums to the finish kernel, which needs whole heads)
  p.split = (ep == EP_QKV || ep == EP_RESID) && (p.two || (N / 16 + 3) / 4 * p.nrb < 512);
  // split launches keep no running sums, so they take wider column groups:
  // fewer of them, and fewer reads of the activations (one per group)
  p.C = p.split ? (ep == EP_RESID ? 8 : (M2 <= 0 ? 12 : 6)) : (ep == EP_RESID || ep == EP_QKV ? 4 : 6);
  if (ep == EP_SWIGLU && (N / 16) % 6 != 0) p.C = 4;   // whole gate/up pairs per workgroup
  p.ng = (N / 16 + p.C - 1) / p.C;
  const int ngs = p.ng * (p.split ? NSL : 1);
  p.wgs = (ngs + 7) / 8 * 8 * p.nrb;
  return true;
}

bool gemm_bf16_rows_form(int M, int N, int ep) {
  RowsPlan rp;
  return rows_plan(M, 0, N, ep, rp);
}

int gemm_bf16_split_slices(int M, int M2, int N, int ep) {
  if (M2 < 0) M2 = 0;
  RowsPlan rp;
  if (rows_plan(M, M2, N, ep, rp)) return rp.split ? NSL : 0;
  int rpw = gemm_rows_per_wg(M, M2);
  int gy = (M + rpw - 1) / rpw + (M2 + rpw - 1) / rpw;
  // QKV takes 64-row tiles where 128-row tiles give fewer than 192
  // workgroups (the launch below makes the same choice)
  if (ep == EP_QKV && rpw == 128 && (N / 128) * gy < 192) {
    rpw = 64;
    gy = (M + rpw - 1) / rpw + (M2 + rpw - 1) / rpw;
  }
  return (N / 128) * gy >= (ep == EP_RESID ? 256 : 128) ? 0 : NSL;
}

// The launch shape launch_gemm_bf16 picks for a GEMM (row tiles, waves per
// workgroup, K split or not, column tiles per wave, workgroups).  Shared by
// the launcher and the measurement query, so the two cannot disagree.
struct GemmPlan { int MT, WV, split, CT, wgs; };

static GemmPlan gemm_plan(int M, int M2, int N, int ep) {
  GemmPlan p{};
  if (M2 < 0) M2 = 0;
  const bool wide = gemm_bf16_split_slices(M, M2, N, ep) == 0;
  const int wv = (ep == EP_SWIGLU && (N / 16) % 6 == 0 && gemm_mt(M, M2) <= 3) ? 6 : 8;
  // tall row tiles for unsplit launches other than gate/up (which takes two
  // column tiles per wave at 128 rows instead: measured faster)
  int MT = wide && ep != EP_SWIGLU ? gemm_mt_tall(M, M2, N / (16 * wv)) : gemm_mt(M, M2);
  // gate/up, and split O / down launches, at 128-row tiles (two column
  // tiles per wave): 144-row tiles where they pad fewer rows (528 rows:
  // 4 x 144 instead of 5 x 128)
  if ((wide ? ep == EP_SWIGLU : ep == EP_RESID) && MT == 8 && M2 == 0 && rows144_pad_less(M))
    MT = 9;
  // QKV (48 column groups at Qwen3-8B width) with 128-row tiles: 64-row
  // tiles when 128 would leave fewer than 192 workgroups.  Measured: 264 + 8
  // draft rows 144 -> 240 workgroups, 2.81 -> 2.02 ms per step; 512 + 16
  // rows (240 workgroups) slower with 64-row tiles, 2.89 -> 3.65 ms.
  if (wide && ep == EP_QKV && MT == 8 && (N / 128) * ((M + 127) / 128 + (M2 + 127) / 128) < 192)
    MT = 4;
  const int rpw = MT > 4 ? MT * 16 : 64;
  const int gy = (M + rpw - 1) / rpw + (M2 + rpw - 1) / rpw;
  p.MT = MT;
  p.split = !wide;
  if (!wide) {
    p.WV = (ep == EP_RESID && (MT == 8 || MT == 9)) ? 4 : 8;
    p.CT = p.WV == 4 ? 2 : 1;
    p.wgs = N / 128 * NSL * gy;
  } else if ((MT == 8 || MT == 9) && ep == EP_SWIGLU) {
    p.WV = 4; p.CT = 2; p.wgs = N / 128 * gy;
  } else {
    p.WV = (ep == EP_SWIGLU && wv == 6) ? 6 : 8;
    p.CT = 1;
    p.wgs = N / (16 * p.WV) * gy;
  }
  return p;
}

extern "C" int orthrus_gemm_plan(int32_t m, int32_t m2, int32_t n, int32_t k, int32_t epilogue,
                                 int32_t* plan) {
  if (!plan || m < 0 || m2 < 0 || m + m2 < 1 || n < 128 || n % 128 || k < 256 || k % 256 ||
      epilogue < EP_RESID || epilogue > EP_QKV)
    return ORTHRUS_EINVAL;
  RowsPlan rp;
  if (rows_plan(m, m2, n, epilogue, rp)) {
    plan[0] = rp.tb; plan[1] = 4; plan[2] = rp.split;
    plan[3] = rp.C; plan[4] = rp.wgs; plan[5] = 1 + rp.two;
    return ORTHRUS_OK;
  }
  const GemmPlan p = gemm_plan(m, m2, n, epilogue);
  plan[0] = p.MT; plan[1] = p.WV; plan[2] = p.split; plan[3] = p.CT; plan[4] = p.wgs; plan[5] = 0;
  return ORTHRUS_OK;
}

void launch_qkv_finish_bf16(const GemmArgs& a, hipStream_t s) {
  const int rows = (a.M > 0 ? a.M : 0) + (a.M2 > 0 ? a.M2 : 0);
  if (rows > 0) hipLaunchKernelGGL(k_qkv_finish_bf16<NSL>, dim3(rows, a.N / 128), dim3(64), 0, s, a);
}

// Shape rules: N a multiple of 128, K a multiple of 256 (8 slices of whole
// k-blocks).  A second segment (W2, M2, row02: same N, K and input buffer)
// runs in the same launch; the argmax epilogue takes one segment only.
void launch_gemm_bf16(const GemmArgs& a0, hipStream_t s) {
  GemmArgs a = a0;
  if (!a.W2 || a.M2 <= 0) { a.W2 = nullptr; a.M2 = 0; }
  if (a.M <= 0 && a.M2 <= 0) return;
  RowsPlan rp;
  if (rows_plan(a.M, a.M2, a.N, a.ep, rp)) {
    a.tnrb = rp.nrb; a.ttb = rp.tb; a.tng = rp.ng;
    const dim3 g(rp.wgs), b(256);
    switch (a.ep) {
      case EP_SWIGLU:
        if (rp.C == 6) gemm_launch(k_gemm_rows<6, EP_SWIGLU, false, false>, g, b, s, a);
        else gemm_launch(k_gemm_rows<4, EP_SWIGLU, false, false>, g, b, s, a);
        break;
      case EP_ARGMAX:
        gemm_launch(k_gemm_rows<6, EP_ARGMAX, false, false>, g, b, s, a);
        hipLaunchKernelGGL(k_amax_rows, dim3(a.M), dim3(64), 0, s, a);
        break;
      case EP_RESID:
        if (!rp.split) gemm_launch(k_gemm_rows<4, EP_RESID, false, false>, g, b, s, a);
        else if (rp.two) gemm_launch(k_gemm_rows<8, EP_RESID, true, true>, g, b, s, a);
        else gemm_launch(k_gemm_rows<8, EP_RESID, true, false>, g, b, s, a);
        break;
      default:
        if (!rp.split) {
          gemm_launch(k_gemm_rows<4, EP_QKV, false, false>, g, b, s, a);
          hipLaunchKernelGGL(k_qkv_finish_bf16<1>, dim3(a.M + a.M2, a.N / 128), dim3(64), 0, s, a);
          break;
        }
        if (rp.two) gemm_launch(k_gemm_rows<6, EP_QKV, true, true>, g, b, s, a);
        else gemm_launch(k_gemm_rows<12, EP_QKV, true, false>, g, b, s, a);
        if (!a.defer_finish) launch_qkv_finish_bf16(a, s);
        break;
    }
    return;
  }
  const GemmPlan plan = gemm_plan(a.M, a.M2, a.N, a.ep);
  const bool wide = !plan.split;
  const int MT = plan.MT;
  const int wv = plan.WV == 6 ? 6 : 8;
  const int rpw = MT > 4 ? MT * 16 : 64;         // rows per workgroup
  a.gy0 = (a.M + rpw - 1) / rpw;
  const dim3 gy(1, a.gy0 + (a.M2 + rpw - 1) / rpw);
  a.gyt = gy.y;
  a.flat = 0;
  if (!wide) {
    const dim3 grid(a.N / 128 * NSL, gy.y);
    switch (a.ep) {
      case EP_RESID:
        // 128- and 144-row tiles: two column tiles per wave
        if (MT == 8) gemm_launch(k_gemm_bf16<8, EP_RESID, 4, true, 2>, grid, dim3(256), s, a);
        else if (MT == 9) gemm_launch(k_gemm_bf16<9, EP_RESID, 4, true, 2>, grid, dim3(256), s, a);
        else dispatch_mt<EP_RESID, 8, true>(MT, grid, a, s);
        break;
      case EP_SWIGLU: dispatch_mt<EP_SWIGLU, 8, true>(MT, grid, a, s); break;
      case EP_QKV:
        dispatch_mt<EP_QKV, 8, true>(MT, grid, a, s);
        if (!a.defer_finish) launch_qkv_finish_bf16(a, s);
        break;
      default: dispatch_mt<EP_ARGMAX, 8, true>(MT, grid, a, s); break;
    }
    return;
  }
  // several row blocks with a column-group count divisible by 8: 1-D grid
  // with each column group's row blocks on one XCD (see the kernel)
  auto grid_of = [&](int ngroups) {
    a.flat = gy.y > 1 && ngroups % 8 == 0;
    return a.flat ? dim3(ngroups * gy.y, 1) : dim3(ngroups, gy.y);
  };
  if ((MT == 8 || MT == 9) && a.ep == EP_SWIGLU) {   // 128 / 144-row tiles: two column tiles per wave
    const dim3 g = grid_of(a.N / 128);
    dispatch_ct2<EP_SWIGLU>(MT, g, a, s);
    return;
  }
  switch (a.ep) {
    case EP_SWIGLU:
      // 96-column workgroups when they divide N: the Qwen3-8B gate/up GEMM
      // (N = 24576) then has exactly one workgroup per compute unit
      if (wv == 6) {
        const dim3 g = grid_of(a.N / 96);
        dispatch_mt<EP_SWIGLU, 6, false>(MT, g, a, s);
      } else {
        const dim3 g = grid_of(a.N / 128);
        dispatch_mt<EP_SWIGLU, 8, false>(MT, g, a, s);
      }
      break;
    case EP_RESID: { const dim3 g = grid_of(a.N / 128); dispatch_mt<EP_RESID, 8, false>(MT, g, a, s); break; }
    case EP_QKV: { const dim3 g = grid_of(a.N / 128); dispatch_mt<EP_QKV, 8, false>(MT, g, a, s); break; }
    default: { const dim3 g = grid_of(a.N / 128); dispatch_mt<EP_ARGMAX, 8, false>(MT, g, a, s); break; }
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
