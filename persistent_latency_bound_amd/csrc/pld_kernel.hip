// Persistent batch-1 decode: one launch runs every stage of a decode layer (and, for
// decode_layers_persistent, every layer of every token) with all workgroups resident.
//
// The design follows the idea of TileRT's persistent "Engine Kernel" (InferenceX,
// "Ultra-High Interactivity on NVIDIA GPUs? TileRT on InferenceX", section "But What
// Exactly is TileRT?"): the host launches once; stages are chained by device-side
// dependencies rather than kernel boundaries; activations stay on chip (LDS) or move
// through the device coherence point rather than being re-staged by separate kernels.
// What is specific to MI355X here:
//  * one 512-thread workgroup per CU (256 CUs in 8 XCDs), each owning a static slice of
//    every stage (rows of each weight matrix, a KV chunk of one kv head, a slice of the
//    expert rows) fixed by the launch geometry — the ahead-of-time schedule of the
//    article's "Why Is TileRT Development Slow?" section, computed from the workgroup id;
//  * weights stream from HBM with 16-byte non-temporal loads, several rows in flight
//    per wave, and the first rows of the next stage are issued before the dependency
//    wait (static weights only; activations after the wait — the ordering fix reported
//    in the vLLM Kimi K3 backend article, "Agent-written kernels face evidence gates");
//  * cross-workgroup dependencies use per-XCD then global counters and write-through
//    agent-scope stores (see pld_device.hpp for the measured choice);
//  * attention is split over KV chunks (one kv head per group of workgroups) and merged
//    by the group's last arriver, which is the single-GPU form of the "attention output
//    partials ... all-reduce ... residual" chain of the vLLM article ("Four changes
//    drive the gains");
//  * the shared expert runs while the router top-k is pending, as the same article
//    describes for its side stream.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <new>
#include <vector>

#include "../../include/pld.h"
#include "pld_device.hpp"

namespace pld {

// ------------------------------------------------------------------ shared structs
enum Stage { S_QKV = 0, S_H2 = 1, S_RT = 2, S_M = 3, S_OUT = 4, S_ATT = 5, NSTG = 8 };
enum { ST_CODE = 0, ST_STAGE = 1, ST_LAYER = 2, ST_TOKEN = 3, ST_WG = 4, ST_ABORT = 8 };
// device trace: wall-clock stamps per (step, workgroup)
enum TraceSlot {
  TR_START = 0, TR_X_READY, TR_QKV_DONE, TR_ATT_READY, TR_ATT_DONE, TR_O_READY, TR_WO_DONE, TR_H2_READY,
  TR_RT_READY, TR_FFN_DONE, TR_M_READY, TR_DOWN_DONE, TR_ATT_Q = 12, TR_ATT_SOFTMAX = 13, TR_ATT_PARTIAL = 14,
  TR_ATT_MERGED = 15, TR_TOPK = 16, TR_ROUTED_GEMV = 17, TR_M_STORED = 18, TR_DOWN_GEMV = 19, TR_DOWN_EPI = 20,
  TR_QKV_GEMV = 21, TR_SHARED_GEMV = 22, TR_X_COPIED = 23, TR_X_NORMED = 24, TR_MERGE_FLAG = 25,
  TR_MERGE_COPIED = 26, TR_RT_LOGIT = 27, TR_O_COPIED = 28, TR_M_COPIED = 29, TR_ATT_SCORES = 30, TR_SLOTS = 32
};

struct KCfg {
  int attn, wfmt, H, nh, nkv, hd, q_lora, kv_lora, rope, nope, vdim, ih, idim, itopk;
  int ffn, inter, E, topk, nshared, router, max_seq, vocab;
  double eps;
  int slots;   // expert slots used per token (routed + shared), 1 for a dense FFN
  int G;       // q heads per kv head
  int cpg;     // attention chunks per kv head = workgroups per kv head
  int chmax;   // max tokens in one attention chunk
  int act_floats, stage_words, outb_floats;
  int nwg;
};

struct DLayer {
  const float *attn_norm, *ffn_norm, *q_norm, *kv_norm;
  DMat wq, wk, wv, wo, w_dq, w_uq, w_dkv, w_uk, w_uv, w_qi, w_w, w_ki;
  const uint16_t* router;
  const float* router_bias;
  DMat w_gate, w_up, w_down;
  size_t gu_slot_bytes, gu_slot_scales, dn_slot_bytes, dn_slot_scales;
  uint16_t *kc, *vc, *lat;
  uint8_t* icodes;
  float* iscales;
};

struct WsOff {
  size_t ctr_xcd, ctr_glob, ctr_grp, ctr_att, status, xbuf, q, part, o, h2, logits, sel, gates, m, a_dbg,
      b_dbg, rope, layers, total;
};

struct KArgs {
  KCfg c;
  uint8_t* ws;
  WsOff off;
  int n_layers, n_tokens, pos0, layer0;
  uint32_t step0;
  const uint16_t* in_hidden;
  uint16_t* out_hidden;
  long long budget;
  uint64_t* trace;     // [trace_steps][nwg][TR_SLOTS] or null
  int trace_steps;
};

// ------------------------------------------------------------------ device context
struct Ctx {
  long long budget;   // watchdog budget of one wait, in wall-clock ticks
  int w, nwg;
  uint32_t *ctr_xcd, *ctr_glob, *ctr_grp, *ctr_att, *status;
  int layer, token;
};

template <typename T>
__device__ __forceinline__ T* wsp(const KArgs& a, size_t off) {
  return reinterpret_cast<T*>(a.ws + off);
}

// Cold path: record the first expired wait and raise the abort flag.
__device__ __noinline__ void raise_timeout(uint32_t* status, int stage, int layer, int token, int w) {
  uint32_t expected = 0;
  if (__hip_atomic_compare_exchange_strong(gp(status + ST_CODE), &expected, (uint32_t)(int32_t)PLD_E_DEVICE_TIMEOUT,
                                           __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    st_u32(status + ST_STAGE, (uint32_t)stage);
    st_u32(status + ST_LAYER, (uint32_t)layer);
    st_u32(status + ST_TOKEN, (uint32_t)token);
    st_u32(status + ST_WG, (uint32_t)w);
  }
  st_u32(status + ST_ABORT, 1u);
}

// Thread 0 spins (bounded) until *ctr reaches target; every thread gets the verdict.
__device__ __forceinline__ bool spin_until(Ctx& cx, const uint32_t* ctr, uint32_t target, int stage) {
  int failed = 0;
  if (threadIdx.x == 0 && (int)(ld_u32(ctr) - target) < 0) {
    const long long deadline = wall_clock64() + cx.budget;
    int n = 0;
    while ((int)(ld_u32(ctr) - target) < 0) {
      if ((++n & 15) == 0) {
        if (ld_u32(cx.status + ST_ABORT)) { failed = 1; break; }
        if (wall_clock64() > deadline) { raise_timeout(cx.status, stage, cx.layer, cx.token, cx.w); failed = 1; break; }
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  return !__syncthreads_or(failed);
}

// Publish: every wave waits for its write-through stores, then one thread counts this
// workgroup in its XCD group; the group's last arriver counts the group globally.
// Participants are workgroups [0, n_part).
__device__ __forceinline__ void arrive(Ctx& cx, int stage, uint32_t k1, int n_part) {
  vm_wait();
  __syncthreads();
  if (threadIdx.x == 0 && cx.w < n_part) {
    const int x = cx.w & (NXCD - 1);
    const uint32_t per = (uint32_t)((n_part - x + NXCD - 1) / NXCD);
    const uint32_t old = atomic_add_u32(cx.ctr_xcd + (stage * NXCD + x) * CTR_STRIDE, 1u);
    if (old + 1u == k1 * per) atomic_add_u32(cx.ctr_glob + stage * CTR_STRIDE, 1u);
  }
}
__device__ __forceinline__ bool wait_all(Ctx& cx, int stage, uint32_t k1, int n_part) {
  const uint32_t groups = (uint32_t)min(NXCD, n_part);
  return spin_until(cx, cx.ctr_glob + stage * CTR_STRIDE, k1 * groups, stage);
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// In-place RMSNorm of act[0..n): act = fp32((act * r) * gamma), r = 1/sqrt(sum(act^2)/n + eps)
// with the statistics in fp64 (bf16 and fp32 squares are exact in fp64).
__device__ __forceinline__ void rmsnorm_inplace(float* act, const float* __restrict__ gamma, int n, double eps,
                                                double* red) {
  double ss = 0.0;
  for (int i = threadIdx.x; i < n; i += BLOCK) ss += (double)act[i] * (double)act[i];
  ss = block_sum(ss, red);
  const double r = 1.0 / sqrt(ss / (double)n + eps);
  const PLD_GLOBAL float* g = gp(gamma);
  for (int i = threadIdx.x; i < n; i += BLOCK) act[i] = (float)(((double)act[i] * r) * (double)g[i]);
  __syncthreads();
}

// This thread's elements i = threadIdx.x + k*BLOCK of a length-N fp32 vector, held in
// registers. Small static vectors (norm weights) are loaded this way BEFORE a stage's
// weight prefetch is issued, so they sit at the front of the wave's in-order load queue
// instead of behind ~tens of KB of weight loads.
template <int N>
struct RegVec {
  static constexpr int K = (N + BLOCK - 1) / BLOCK;
  float v[K];
  __device__ __forceinline__ void load(const float* p) {
    const PLD_GLOBAL float* g = gp(p);
#pragma unroll
    for (int k = 0; k < K; k++) {
      const int i = threadIdx.x + k * BLOCK;
      v[k] = i < N ? g[i] : 0.f;
    }
  }
};
// rmsnorm_inplace with the weights in registers (same arithmetic, same summation order)
template <int N>
__device__ __forceinline__ void rmsnorm_reg(float* act, const RegVec<N>& gam, double eps, double* red) {
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < RegVec<N>::K; k++) {
    const int i = threadIdx.x + k * BLOCK;
    if (i < N) ss += (double)act[i] * (double)act[i];
  }
  ss = block_sum(ss, red);
  const double r = 1.0 / sqrt(ss / (double)N + eps);
#pragma unroll
  for (int k = 0; k < RegVec<N>::K; k++) {
    const int i = threadIdx.x + k * BLOCK;
    if (i < N) act[i] = (float)(((double)act[i] * r) * (double)gam.v[k]);
  }
  __syncthreads();
}

// Weight loads in flight per lane for each GEMV stage (16-byte loads). Deep prefetch
// keeps HBM busy, but every load queued ahead of a latency-critical access (a counter
// poll, an activation copy) delays it: the queue drains at the lane's share of HBM
// bandwidth. The depths below were chosen by measurement.
#ifndef PLD_IF_QKV
#define PLD_IF_QKV 8
#endif
#ifndef PLD_IF_WO
#define PLD_IF_WO 8
#endif
#ifndef PLD_IF_SHARED
#define PLD_IF_SHARED 8
#endif
#ifndef PLD_IF_ROUTED
#define PLD_IF_ROUTED 8
#endif
#ifndef PLD_IF_DOWN
#define PLD_IF_DOWN 8
#endif

// ------------------------------------------------------------------ LDS layout
struct Lds {
  float* act;        // [act_floats]   activation vector / attention scratch / merge staging
  uint32_t* stage;   // [stage_words]  raw bf16-pair words of the incoming hidden state
  float* outb;       // [outb_floats]  GEMV row results
  float* outc;       // [outb_floats]
  float* xres;       // [outb_floats]  this workgroup's rows of the layer input (for the residual)
  double* red;       // [16]
  int* isel;         // [32]
  float* fgate;      // [32]
  int* flag;         // [8]
  RowSeg* segs;      // [MAX_SEGS] GEMV segment list of the current stage
};
__device__ __forceinline__ Lds carve(float* base, const KCfg& c) {
  Lds L;
  L.act = base;
  L.stage = reinterpret_cast<uint32_t*>(base + c.act_floats);
  L.outb = reinterpret_cast<float*>(L.stage + c.stage_words);
  L.outc = L.outb + c.outb_floats;
  L.xres = L.outc + c.outb_floats;
  L.red = reinterpret_cast<double*>(L.xres + c.outb_floats);
  L.isel = reinterpret_cast<int*>(L.red + 16);
  L.fgate = reinterpret_cast<float*>(L.isel + 32);
  L.flag = reinterpret_cast<int*>(L.fgate + 32);
  L.segs = reinterpret_cast<RowSeg*>(L.flag + 8);
  return L;
}
__host__ __device__ inline size_t lds_bytes_for(int act_floats, int stage_words, int outb_floats) {
  return (size_t)4 * (act_floats + stage_words + 3 * outb_floats) + 8 * 16 + 4 * 32 + 4 * 32 + 4 * 8 +
         sizeof(RowSeg) * MAX_SEGS;
}

// Publishes a segment list to the workgroup (the previous list must be out of use).
__device__ __forceinline__ void seg_begin() { __syncthreads(); }
__device__ __forceinline__ void seg_set(Lds& L, int i, const uint8_t* w, const float* sc, int n, int srow, int act_off,
                                        float alpha) {
  if (threadIdx.x == 0) {
    RowSeg& S = L.segs[i];
    S.w = w; S.s = sc; S.n = n; S.srow = srow; S.act_off = act_off; S.alpha = alpha;
  }
}
__device__ __forceinline__ void seg_end() { __syncthreads(); }

// ------------------------------------------------------------------ compiled layer shapes
// One kernel is compiled per supported layer shape, so every reduction length, head
// size and expert width is a compile-time constant: each GEMV call site gets exactly one
// lane layout, and the whole step inlines into the kernel (no device calls on the hot
// path). Row counts that vary at run time (experts, top-k, cache length) stay runtime.
// ATT_NB = K row passes and ATT_NV V tokens per wave held in registers per attention batch.
template <int H_, int NH_, int NKV_, int HD_, int INTER_, bool FP8_, bool MOE_, int ATT_NB_, int ATT_NV_>
struct GqaShape {
  static constexpr int H = H_, NH = NH_, NKV = NKV_, HD = HD_, INTER = INTER_, ATT_NB = ATT_NB_, ATT_NV = ATT_NV_;
  static constexpr int G = NH / NKV, ODIM = NH * HD;
  static constexpr bool FP8 = FP8_, MOE = MOE_;
  static_assert(H % 2 == 0 && ODIM % 2 == 0, "hidden sizes must be even");
};

// Per-(token, layer) state of one workgroup.
struct Step {
  const DLayer* Ly;
  const uint16_t* in_hidden;   // caller's bf16 input for the first step of the launch, else null
  uint32_t k1;                 // step number + 1 (counter epoch)
  bool first;                  // first step of the launch
  int pos;
  int idx;                     // step index within the launch (trace row)
};

__device__ __forceinline__ void stamp(const KArgs& a, const Ctx& cx, const Step& st, int slot) {
  if (a.trace && st.idx < a.trace_steps && threadIdx.x == 0)
    gp(a.trace)[((size_t)st.idx * cx.nwg + cx.w) * TR_SLOTS + slot] = wall_clock64();
}

// Rows [r0, r1) of an H-row stage for this workgroup, split in pairs (the hidden state
// moves between workgroups as packed bf16 pairs).
__device__ __forceinline__ void hrows(int H, int nwg, int w, int* r0, int* r1) {
  *r0 = 2 * split_at(H / 2, nwg, w);
  *r1 = 2 * split_at(H / 2, nwg, w + 1);
}

// ------------------------------------------------------------------ stage: RMSNorm + QKV + RoPE + cache append
template <class SH>
__device__ __forceinline__ bool stage_qkv_gqa(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  constexpr int HD = SH::HD;
  const int w = cx.w, nwg = cx.nwg, pos = st.pos;
  constexpr int qR = SH::NH * HD, kR = SH::NKV * HD, R = qR + 2 * kR;
  constexpr int P = R / 2;
  const int r0 = 2 * split_at(P, nwg, w), r1 = 2 * split_at(P, nwg, w + 1);
  int h0, h1;
  hrows(SH::H, nwg, w, &h0, &h1);
  RegVec<SH::H> gam;
  gam.load(Ly.attn_norm);
  bool pending = true;   // the input wait + RMSNorm has not run yet
  auto pre_x = [&]() -> bool {
    if (!pending) return true;
    pending = false;
    if (!st.first && !wait_all(cx, S_OUT, st.k1 - 1, nwg)) return false;
    stamp(a, cx, st, TR_X_READY);
    // stage the bf16 pairs of x, keep this workgroup's residual rows, expand to fp32
    if (st.first) {
      const PLD_GLOBAL uint32_t* src = gp(reinterpret_cast<const uint32_t*>(st.in_hidden));
      for (int i = threadIdx.x; i < SH::H / 2; i += BLOCK) L.stage[i] = src[i];
    } else {
      coh_copy_to_lds(L.stage, wsp<uint32_t>(a, a.off.xbuf), SH::H / 2);
    }
    __syncthreads();
    stamp(a, cx, st, TR_X_COPIED);
    for (int i = threadIdx.x; i < SH::H / 2; i += BLOCK) {
      const uint32_t v = L.stage[i];
      L.act[2 * i] = bf_lo(v);
      L.act[2 * i + 1] = bf_hi(v);
    }
    __syncthreads();
    for (int r = h0 + threadIdx.x; r < h1; r += BLOCK) L.xres[r - h0] = L.act[r];
    rmsnorm_reg<SH::H>(L.act, gam, c.eps, L.red);
    stamp(a, cx, st, TR_X_NORMED);
    if (w == 0)
      for (int i = threadIdx.x; i < SH::H; i += BLOCK) st_f32(wsp<float>(a, a.off.a_dbg) + i, L.act[i]);
    return true;
  };
  {
    // one pipelined pass over this workgroup's rows of [W_q; W_k; W_v]
    const DMat* mats[3] = {&Ly.wq, &Ly.wk, &Ly.wv};
    const int seg0[4] = {0, qR, qR + kR, R};
    constexpr size_t RB = (size_t)SH::H * (SH::FP8 ? 1 : 2);
    seg_begin();
    int ns = 0;
#pragma unroll
    for (int m = 0; m < 3; m++) {
      const int lo = max(r0, seg0[m]), hi = min(r1, seg0[m + 1]);
      if (lo < hi) {
        seg_set(L, ns, mats[m]->w + (size_t)(lo - seg0[m]) * RB, mats[m]->s, hi - lo, lo - seg0[m], 0, 1.f);
        ns++;
      }
    }
    seg_end();
    if (!gemv_list<SH::FP8, SH::H, PLD_IF_QKV>(L.segs, ns, L.act, L.outb, OUT_STORE, pre_x)) return false;
  }
  stamp(a, cx, st, TR_QKV_GEMV);
  if (!pre_x()) return false;
  __syncthreads();
  const PLD_GLOBAL float* rope = gp(wsp<float>(a, a.off.rope)) + (size_t)pos * HD;   // (cos, sin) pairs
  float* qw = wsp<float>(a, a.off.q);
  for (int p = r0 / 2 + threadIdx.x; p < r1 / 2; p += BLOCK) {
    const int r = 2 * p;
    float v0 = L.outb[r - r0], v1 = L.outb[r + 1 - r0];
    if (r < qR + kR) {
      const int d = (r < qR ? r : r - qR) % HD;
      const float cs = rope[d], sn = rope[d + 1];
      const float x0 = v0 * cs - v1 * sn, x1 = v0 * sn + v1 * cs;
      v0 = x0;
      v1 = x1;
    }
    if (r < qR) {
      st_u64(reinterpret_cast<uint64_t*>(qw + r), (uint64_t)__float_as_uint(v0) | ((uint64_t)__float_as_uint(v1) << 32));
    } else {
      const bool isk = r < qR + kR;
      const int rr = isk ? r - qR : r - qR - kR;
      const int head = rr / HD, d = rr % HD;
      uint16_t* dst = (isk ? Ly.kc : Ly.vc) + ((size_t)head * c.max_seq + pos) * HD + d;
      st_u32(reinterpret_cast<uint32_t*>(dst), f32_to_bf16(v0) | (f32_to_bf16(v1) << 16));
    }
  }
  arrive(cx, S_QKV, st.k1, nwg);
  stamp(a, cx, st, TR_QKV_DONE);
  return true;
}

// ------------------------------------------------------------------ attention (GQA)
// One workgroup = one (kv head g, token chunk) pair. Scores for the G query heads of
// the group, chunk-local softmax, P.V, then a partial (m, l, acc[HD]) per head. The
// group's last arriver merges the partials into o.
//  * scores: 16-byte K loads, HD/8 lanes per token row, ATT_NB row passes held in
//    registers; the per-token dot is reduced with DPP moves inside each 16-lane row;
//  * P.V: each wave owns a contiguous token range and each lane HD/64 dims, so the sum
//    over tokens needs no lane exchange, only one cross-wave pass through LDS;
//  * the static history rows of the first batch (K and V) are issued before the wait
//    for this step's q/k/v; rows written in this launch are read coherently after it.
template <class SH>
__device__ __forceinline__ bool attention_gqa(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  const uint32_t k1 = st.k1;
  constexpr int HD = SH::HD, G = SH::G, NB = SH::ATT_NB, NV = SH::ATT_NV;
  constexpr int LPT = HD / 8;          // lanes per token row in the score pass (16 bytes each)
  constexpr int TPW = 64 / LPT;        // tokens per wave pass
  constexpr int PASS = NWAVES * TPW;   // tokens per workgroup pass
  constexpr int DPL = HD / 64;         // dims per lane in the P.V pass
  static_assert(DPL == 1 || DPL == 2, "head dim 64 or 128");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int dl = lane % LPT, tl = lane / LPT;
  const int cpg = c.cpg;
  const int g = cx.w / cpg, ch = cx.w % cpg;
  if (g < SH::NKV) {   // workgroups past the last group only take part in the final arrive
  const int T = st.pos + 1;
  const int t0 = split_at(T, cpg, ch), t1 = split_at(T, cpg, ch + 1), n = t1 - t0;
  const int tw = (n + NWAVES - 1) / NWAVES;             // P.V tokens per wave
  const int pv0 = min(n, wave * tw), pv1 = min(n, pv0 + tw);
  const uint16_t* kbase = Ly.kc + (size_t)g * c.max_seq * HD + dl * 8;
  const uint16_t* vbase = Ly.vc + (size_t)g * c.max_seq * HD + lane * DPL;
  const int fresh = a.pos0;   // rows >= fresh were written inside this launch: coherent loads only
  auto tok = [&](int tb0, int b) { return tb0 + b * PASS + wave * TPW + tl; };
  auto k_static = [&](int t) -> uint4 {
    return (t < n && t0 + t < fresh) ? ld_g16(kbase + (size_t)(t0 + t) * HD) : make_uint4(0u, 0u, 0u, 0u);
  };
  auto k_fresh = [&](int t) -> uint4 {
    const uint64_t* q = reinterpret_cast<const uint64_t*>(kbase + (size_t)(t0 + t) * HD);
    const uint64_t x = ld_u64(q), y = ld_u64(q + 1);
    return make_uint4((uint32_t)x, (uint32_t)(x >> 32), (uint32_t)y, (uint32_t)(y >> 32));
  };
  // V element(s) of this lane for token t (DPL bf16 values packed in a word)
  auto v_static = [&](int t) -> uint32_t {
    if (t >= pv1 || t0 + t >= fresh) return 0u;
    const uint16_t* p = vbase + (size_t)(t0 + t) * HD;
    if constexpr (DPL == 2) return *(const PLD_GLOBAL uint32_t*)(p);
    else return (uint32_t)(*(const PLD_GLOBAL uint16_t*)(p));
  };
  auto v_fresh = [&](int t) -> uint32_t {
    const uint16_t* p = vbase + (size_t)(t0 + t) * HD;
    if constexpr (DPL == 2) return ld_u32(reinterpret_cast<const uint32_t*>(p));
    else {
      const uint32_t w2 = ld_u32(reinterpret_cast<const uint32_t*>(p - (lane & 1)));
      return (lane & 1) ? (w2 >> 16) : (w2 & 0xffffu);
    }
  };
  uint4 kb[NB];
  uint32_t vb[NV];
#pragma unroll
  for (int b = 0; b < NB; b++) kb[b] = k_static(tok(0, b));
#pragma unroll
  for (int b = 0; b < NV; b++) vb[b] = v_static(pv0 + b);
  if (!wait_all(cx, S_QKV, k1, cx.nwg)) return false;
  stamp(a, cx, st, TR_ATT_READY);

  const uint64_t* qg = reinterpret_cast<const uint64_t*>(wsp<float>(a, a.off.q) + (size_t)g * G * HD + dl * 8);
  const float scale = 1.0f / sqrtf((float)HD);
  float qr[G][8];
#pragma unroll
  for (int h = 0; h < G; h++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint64_t v = ld_u64(qg + h * HD / 2 + j);
      qr[h][2 * j] = __uint_as_float((uint32_t)v) * scale;
      qr[h][2 * j + 1] = __uint_as_float((uint32_t)(v >> 32)) * scale;
    }
  stamp(a, cx, st, TR_ATT_Q);
  float* sc = L.act;                               // [G][chmax]
  float* red2 = L.act + G * c.chmax;               // [NWAVES][G][HD]
  float* ml = red2 + NWAVES * G * HD;              // [2G]
  // ---- pass 1: scores
  for (int tb0 = 0; tb0 < n; tb0 += NB * PASS) {
#pragma unroll
    for (int b = 0; b < NB; b++) {
      const int t = tok(tb0, b);
      if (tb0 > 0) kb[b] = k_static(t);
      if (t < n && t0 + t >= fresh) kb[b] = k_fresh(t);
    }
#pragma unroll
    for (int b = 0; b < NB; b++) {
      const int t = tok(tb0, b);
      const uint4 kv = kb[b];
      const float kf[8] = {bf_lo(kv.x), bf_hi(kv.x), bf_lo(kv.y), bf_hi(kv.y),
                           bf_lo(kv.z), bf_hi(kv.z), bf_lo(kv.w), bf_hi(kv.w)};
#pragma unroll
      for (int h = 0; h < G; h++) {
        float sh = 0.f;
#pragma unroll
        for (int j = 0; j < 8; j++) sh = fmaf(qr[h][j], kf[j], sh);
        sh = dpp_sum<LPT>(sh);
        if (dl == LPT - 1 && t < n) sc[h * c.chmax + t] = sh;
      }
    }
  }
  stamp(a, cx, st, TR_ATT_SCORES);
  __syncthreads();
  for (int h = wave; h < G; h += NWAVES) {
    float m = -INFINITY;
    for (int t = lane; t < n; t += 64) m = fmaxf(m, sc[h * c.chmax + t]);
    m = wave_max(m);
    float l = 0.f;
    for (int t = lane; t < n; t += 64) {
      const float p = __expf(sc[h * c.chmax + t] - m);
      sc[h * c.chmax + t] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) { ml[2 * h] = m; ml[2 * h + 1] = l; }
  }
  __syncthreads();
  stamp(a, cx, st, TR_ATT_SOFTMAX);
  // ---- pass 2: P.V over this wave's token range, DPL dims per lane
  float acc[G][DPL];
#pragma unroll
  for (int h = 0; h < G; h++)
#pragma unroll
    for (int e = 0; e < DPL; e++) acc[h][e] = 0.f;
  for (int tb = pv0; tb < pv1; tb += NV) {
#pragma unroll
    for (int b = 0; b < NV; b++) {
      const int t = tb + b;
      if (tb > pv0) vb[b] = v_static(t);
      if (t < pv1 && t0 + t >= fresh) vb[b] = v_fresh(t);
    }
#pragma unroll
    for (int b = 0; b < NV; b++) {
      const int t = tb + b;
      if (t < pv1) {
        const float v0 = bf_lo(vb[b]);
        const float v1 = DPL == 2 ? bf_hi(vb[b]) : 0.f;
#pragma unroll
        for (int h = 0; h < G; h++) {
          const float p = sc[h * c.chmax + t];
          acc[h][0] = fmaf(p, v0, acc[h][0]);
          if constexpr (DPL == 2) acc[h][1] = fmaf(p, v1, acc[h][1]);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; h++)
#pragma unroll
    for (int e = 0; e < DPL; e++) red2[(wave * G + h) * HD + lane * DPL + e] = acc[h][e];
  __syncthreads();
  // partial of head h for this chunk: [m, l, acc[0..HD)] at ((g*G + h)*cpg + ch)*(HD+2)
  float* part = wsp<float>(a, a.off.part);
  for (int i = threadIdx.x; i < G * HD / 2; i += BLOCK) {
    const int h = (2 * i) / HD, d = (2 * i) % HD;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int wv = 0; wv < NWAVES; wv++) {
      s0 += red2[(wv * G + h) * HD + d];
      s1 += red2[(wv * G + h) * HD + d + 1];
    }
    st_u64(reinterpret_cast<uint64_t*>(part + ((size_t)(g * G + h) * cpg + ch) * (HD + 2) + 2 + d),
           (uint64_t)__float_as_uint(s0) | ((uint64_t)__float_as_uint(s1) << 32));
  }
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    st_u64(reinterpret_cast<uint64_t*>(part + ((size_t)(g * G + h) * cpg + ch) * (HD + 2)),
           (uint64_t)__float_as_uint(ml[2 * h]) | ((uint64_t)__float_as_uint(ml[2 * h + 1]) << 32));
  }
  // Distributed merge: once all cpg partials of the group are stored, workgroup ch of
  // the group merges dims [d0, d1) of the group's G*HD outputs (flash-decoding rescale:
  // o = sum_c e^(m_c - M) acc_c / sum_c e^(m_c - M) l_c over the chunks with l_c > 0).
  vm_wait();
  __syncthreads();
  stamp(a, cx, st, TR_ATT_PARTIAL);
  if (threadIdx.x == 0) atomic_add_u32(cx.ctr_grp + g * CTR_STRIDE, 1u);
  if (!spin_until(cx, cx.ctr_grp + g * CTR_STRIDE, k1 * (uint32_t)cpg, 9)) return false;
  stamp(a, cx, st, TR_MERGE_FLAG);
  {
    const int d0 = split_at(G * HD, cpg, ch), d1 = split_at(G * HD, cpg, ch + 1), nd = d1 - d0;
    const float* pg = part + (size_t)g * G * cpg * (HD + 2);
    float* mls = L.act;              // [cpg][2] (m, l) of the head of dim d0 .. (two heads at most)
    float* accs = L.act + 4 * cpg;   // [cpg][nd]
    const int h0 = d0 / HD, hlast = (d1 - 1) / HD;
    for (int i = threadIdx.x; i < cpg * nd; i += BLOCK) {
      const int cc = i / nd, j = i % nd, d = d0 + j;
      accs[i] = ld_f32(pg + ((size_t)(d / HD) * cpg + cc) * (HD + 2) + 2 + d % HD);
    }
    for (int i = threadIdx.x; i < cpg * (hlast - h0 + 1); i += BLOCK) {
      const int hh = i / cpg, cc = i % cpg;
      const uint64_t v = ld_u64(reinterpret_cast<const uint64_t*>(pg + ((size_t)(h0 + hh) * cpg + cc) * (HD + 2)));
      mls[2 * i] = __uint_as_float((uint32_t)v);
      mls[2 * i + 1] = __uint_as_float((uint32_t)(v >> 32));
    }
    __syncthreads();
    stamp(a, cx, st, TR_MERGE_COPIED);
    float* obuf = wsp<float>(a, a.off.o) + (size_t)g * G * HD;
    for (int j = threadIdx.x; j < nd; j += BLOCK) {
      const int d = d0 + j;
      const float* ml2 = mls + 2 * cpg * (d / HD - h0);
      float M = -INFINITY;
      for (int cc = 0; cc < cpg; cc++)
        if (ml2[2 * cc + 1] > 0.f) M = fmaxf(M, ml2[2 * cc]);
      float Ls = 0.f, o = 0.f;
      for (int cc = 0; cc < cpg; cc++) {
        const float l = ml2[2 * cc + 1];
        if (l > 0.f) {
          const float f = __expf(ml2[2 * cc] - M);
          Ls += f * l;
          o += f * accs[cc * nd + j];
        }
      }
      st_f32(obuf + d, o / Ls);
    }
  }
  }   // grouped workgroups
  arrive(cx, S_ATT, k1, cx.nwg);
  stamp(a, cx, st, TR_ATT_MERGED);
  stamp(a, cx, st, TR_ATT_DONE);
  return true;
}

// ------------------------------------------------------------------ stage: output projection + residual
template <class SH>
__device__ __forceinline__ bool stage_wo(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  int r0, r1;
  hrows(SH::H, cx.nwg, cx.w, &r0, &r1);
  auto pre_o = [&]() -> bool {
    if (!wait_all(cx, S_ATT, st.k1, cx.nwg)) return false;
    stamp(a, cx, st, TR_O_READY);
    coh_copy_to_lds(reinterpret_cast<uint32_t*>(L.act), wsp<uint32_t>(a, a.off.o), SH::ODIM);
    __syncthreads();
    stamp(a, cx, st, TR_O_COPIED);
    return true;
  };
  {
    const DMat wo = gp(st.Ly)->wo;
    seg_begin();
    seg_set(L, 0, wo.w + (size_t)r0 * SH::ODIM * (SH::FP8 ? 1 : 2), wo.s, r1 - r0, r0, 0, 1.f);
    seg_end();
    if (!gemv_list<SH::FP8, SH::ODIM, PLD_IF_WO>(L.segs, r1 > r0 ? 1 : 0, L.act, L.outb, OUT_STORE, pre_o)) return false;
  }
  __syncthreads();
  float* h2 = wsp<float>(a, a.off.h2);
  for (int r = r0 + 2 * threadIdx.x; r < r1; r += 2 * BLOCK)
    st_u64(reinterpret_cast<uint64_t*>(h2 + r), (uint64_t)__float_as_uint(L.xres[r - r0] + L.outb[r - r0]) |
                                                    ((uint64_t)__float_as_uint(L.xres[r + 1 - r0] + L.outb[r + 1 - r0]) << 32));
  arrive(cx, S_H2, st.k1, cx.nwg);
  stamp(a, cx, st, TR_WO_DONE);
  return true;
}

// ------------------------------------------------------------------ stage: FFN gate/up (+ router)
// Gate/up rows of several (expert, slot, row range) pieces as one GEMV list, then
// m[slot][j] = silu(gate_j . b) * (up_j . b). Each piece contributes a gate segment and
// an up segment; results come back in list order.
struct GuPiece { int expert, slot, j0, j1; };
template <class SH, int INFL, typename Pre>
__device__ __forceinline__ bool gate_up_list(const KArgs& a, const Step& st, Lds& L, const GuPiece* pc, int np, Pre&& pre) {
  const DLayer Ly = *gp(st.Ly);
  constexpr size_t RB = (size_t)SH::H * (SH::FP8 ? 1 : 2);
  seg_begin();
  for (int p = 0; p < np; p++) {
    const size_t bo = (size_t)pc[p].expert * Ly.gu_slot_bytes + (size_t)pc[p].j0 * RB;
    const float* sg = SH::FP8 ? Ly.w_gate.s + (size_t)pc[p].expert * Ly.gu_slot_scales : nullptr;
    const float* su = SH::FP8 ? Ly.w_up.s + (size_t)pc[p].expert * Ly.gu_slot_scales : nullptr;
    seg_set(L, 2 * p, Ly.w_gate.w + bo, sg, pc[p].j1 - pc[p].j0, pc[p].j0, 0, 1.f);
    seg_set(L, 2 * p + 1, Ly.w_up.w + bo, su, pc[p].j1 - pc[p].j0, pc[p].j0, 0, 1.f);
  }
  seg_end();
  if (!gemv_list<SH::FP8, SH::H, INFL>(L.segs, 2 * np, L.act, L.outb, OUT_STORE, pre)) return false;
  __syncthreads();
  float* mbuf = wsp<float>(a, a.off.m);
  int base = 0;
  for (int p = 0; p < np; p++) {
    const int n = pc[p].j1 - pc[p].j0;
    for (int j = threadIdx.x; j < n; j += BLOCK)
      st_f32(mbuf + (size_t)pc[p].slot * SH::INTER + pc[p].j0 + j, silu_f(L.outb[base + j]) * L.outb[base + n + j]);
    base += 2 * n;
  }
  return true;
}

template <class SH>
__device__ __forceinline__ bool stage_ffn(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  const int w = cx.w, nwg = cx.nwg;
  RegVec<SH::H> gam;
  gam.load(Ly.ffn_norm);
  // router workgroups: their router row, loaded ahead of the expert weights
  constexpr int RCH = SH::H / 8, RPT = (RCH + BLOCK - 1) / BLOCK;
  uint4 rrow[SH::MOE ? RPT : 1];
  if constexpr (SH::MOE) {
    if (w < c.E) {
      const uint16_t* rp0 = Ly.router + (size_t)w * SH::H;
#pragma unroll
      for (int k = 0; k < RPT; k++) {
        const int q = threadIdx.x + k * BLOCK;
        rrow[k] = q < RCH ? ld_g16(rp0 + q * 8) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  bool pending = true;
  // wait for h2, RMSNorm it into LDS; router workgroups compute their logit (fp64)
  auto pre_b = [&]() -> bool {
    if (!pending) return true;
    pending = false;
    if (!wait_all(cx, S_H2, st.k1, nwg)) return false;
    stamp(a, cx, st, TR_H2_READY);
    coh_copy_to_lds(reinterpret_cast<uint32_t*>(L.act), wsp<uint32_t>(a, a.off.h2), SH::H);
    __syncthreads();
    rmsnorm_reg<SH::H>(L.act, gam, c.eps, L.red);
    if (w == 0)
      for (int i = threadIdx.x; i < SH::H; i += BLOCK) st_f32(wsp<float>(a, a.off.b_dbg) + i, L.act[i]);
    if constexpr (SH::MOE) {
      if (w < c.E) {
        // logit of expert w (fp64 accumulation) and its selection key: the logit itself
        // (softmax router) or sigmoid(logit) + bias (biased-score router)
        double s = 0.0;
#pragma unroll
        for (int k = 0; k < RPT; k++) {
          const int q = threadIdx.x + k * BLOCK;
          if (q < RCH) s += dot8_bf16_f64(rrow[k], L.act + q * 8);
        }
        s = block_sum(s, L.red);
        if (threadIdx.x == 0) {
          const double key = c.router == PLD_ROUTER_SIGMOID_BIAS
                                 ? (1.0 / (1.0 + exp(-s))) + (double)gp(Ly.router_bias)[w] : s;
          double* lk = wsp<double>(a, a.off.logits) + 2 * w;
          st_u64(reinterpret_cast<uint64_t*>(lk), (uint64_t)__double_as_longlong(s));
          st_u64(reinterpret_cast<uint64_t*>(lk + 1), (uint64_t)__double_as_longlong(key));
        }
        stamp(a, cx, st, TR_RT_LOGIT);
      }
      arrive(cx, S_RT, st.k1, c.E);
    }
    return true;
  };
  const int j0 = split_at(SH::INTER, nwg, w), j1 = split_at(SH::INTER, nwg, w + 1);
  if constexpr (!SH::MOE) {
    const GuPiece pc[1] = {{0, 0, j0, j1}};
    if (!gate_up_list<SH, PLD_IF_SHARED>(a, st, L, pc, j1 > j0 ? 1 : 0, pre_b)) return false;
  } else {
    // shared experts first: they do not depend on the router
    GuPiece pc[2];
    int np = 0;
    for (int sj = 0; sj < c.nshared && j1 > j0; sj++) pc[np++] = {c.E + sj, c.topk + sj, j0, j1};
    if (!gate_up_list<SH, PLD_IF_SHARED>(a, st, L, pc, np, pre_b)) return false;
    if (!pre_b()) return false;
    stamp(a, cx, st, TR_SHARED_GEMV);
    // router top-k (every workgroup computes the same selection)
    if (!wait_all(cx, S_RT, st.k1, c.E)) return false;
    stamp(a, cx, st, TR_RT_READY);
    // top-k by rank: expert e is selected at position rank(e) = #{j : key_j > key_e or
    // (key_j == key_e and j < e)} when that rank is < topk (lowest index wins ties)
    double* lk = reinterpret_cast<double*>(L.outb);   // [E][2] (logit, key); outb is free here
    coh_copy_to_lds(reinterpret_cast<uint32_t*>(lk), wsp<uint32_t>(a, a.off.logits), 4 * c.E);
    __syncthreads();
    const bool sig = c.router == PLD_ROUTER_SIGMOID_BIAS;
    for (int e = threadIdx.x; e < c.E; e += BLOCK) {
      const double ke = lk[2 * e + 1];
      int rank = 0;
      for (int j = 0; j < c.E; j++) {
        const double kj = lk[2 * j + 1];
        rank += (kj > ke) || (kj == ke && j < e);
      }
      if (rank < c.topk) L.isel[rank] = e;
    }
    __syncthreads();
    stamp(a, cx, st, TR_TOPK);
    // gates: softmax over the selected logits, or sigmoid scores normalised over the selection
    double* num = reinterpret_cast<double*>(L.outc);
    if (threadIdx.x < c.topk) {
      const double r = lk[2 * L.isel[threadIdx.x]];
      num[threadIdx.x] = sig ? 1.0 / (1.0 + exp(-r)) : exp(r - lk[2 * L.isel[0]]);
    }
    __syncthreads();
    if (threadIdx.x < c.topk) {
      double gsum = 0.0;
      for (int j = 0; j < c.topk; j++) gsum += num[j];
      L.fgate[threadIdx.x] = (float)(num[threadIdx.x] / gsum);
    }
    __syncthreads();
    if (w == 0 && threadIdx.x < c.topk) {
      st_u32(reinterpret_cast<uint32_t*>(wsp<int>(a, a.off.sel)) + threadIdx.x, (uint32_t)L.isel[threadIdx.x]);
      st_f32(wsp<float>(a, a.off.gates) + threadIdx.x, L.fgate[threadIdx.x]);
    }
    // routed experts: this workgroup's share of the topk*inter (slot, row) pairs, one list
    const int tot = c.topk * SH::INTER;
    const int i0 = split_at(tot, nwg, w), i1 = split_at(tot, nwg, w + 1);
    GuPiece rp[MAX_SEGS / 2];
    int nr = 0;
    for (int s = i0 / SH::INTER; s < c.topk && s * SH::INTER < i1 && nr < MAX_SEGS / 2; s++) {
      const int lo = max(i0, s * SH::INTER) - s * SH::INTER, hi = min(i1, (s + 1) * SH::INTER) - s * SH::INTER;
      if (lo < hi) rp[nr++] = {L.isel[s], s, lo, hi};
    }
    if (!gate_up_list<SH, PLD_IF_ROUTED>(a, st, L, rp, nr, NoPre{})) return false;
  }
  stamp(a, cx, st, TR_M_STORED);
  arrive(cx, S_M, st.k1, nwg);
  stamp(a, cx, st, TR_FFN_DONE);
  return true;
}

// ------------------------------------------------------------------ stage: down projections + residual
template <class SH>
__device__ __forceinline__ bool stage_down(Ctx& cx, const KArgs& a, const Step& st, Lds& L, uint16_t* out_hidden) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  int r0, r1;
  hrows(SH::H, cx.nwg, cx.w, &r0, &r1);
  bool pending = true;
  auto pre_m = [&]() -> bool {
    if (!pending) return true;
    pending = false;
    if (!wait_all(cx, S_M, st.k1, cx.nwg)) return false;
    stamp(a, cx, st, TR_M_READY);
    coh_copy_to_lds(reinterpret_cast<uint32_t*>(L.act), wsp<uint32_t>(a, a.off.m), c.slots * SH::INTER);
    __syncthreads();
    stamp(a, cx, st, TR_M_COPIED);
    return true;
  };
  {
    // all slots' rows [r0, r1) as one list; slot s reads activation m_s
    constexpr size_t RB = (size_t)SH::INTER * (SH::FP8 ? 1 : 2);
    seg_begin();
    for (int s = 0; s < c.slots; s++) {
      const int expert = !SH::MOE ? 0 : (s < c.topk ? L.isel[s] : c.E + (s - c.topk));
      const size_t bo = (size_t)expert * Ly.dn_slot_bytes + (size_t)r0 * RB;
      const float* sd = SH::FP8 ? Ly.w_down.s + (size_t)expert * Ly.dn_slot_scales : nullptr;
      seg_set(L, s, Ly.w_down.w + bo, sd, r1 - r0, r0, s * SH::INTER, 1.f);
    }
    seg_end();
    if (!gemv_list<SH::FP8, SH::INTER, PLD_IF_DOWN>(L.segs, r1 > r0 ? c.slots : 0, L.act, L.outb, OUT_STORE, pre_m))
      return false;
  }
  stamp(a, cx, st, TR_DOWN_GEMV);
  if (!pre_m()) return false;
  __syncthreads();
  // f_r = sum_s gate_s * down_s[r] (fixed slot order)
  {
    const int nr = r1 - r0;
    for (int r = threadIdx.x; r < nr; r += BLOCK) {
      float f = 0.f;
      for (int s = 0; s < c.slots; s++) f += ((!SH::MOE || s >= c.topk) ? 1.0f : L.fgate[s]) * L.outb[s * nr + r];
      L.outc[r] = f;
    }
  }
  __syncthreads();
  // out = h2 + f, rounded to bf16; h2 rows are this workgroup's own (same pair split)
  const uint64_t* h2 = reinterpret_cast<const uint64_t*>(wsp<float>(a, a.off.h2));
  uint32_t* xb = wsp<uint32_t>(a, a.off.xbuf);
  for (int r = r0 + 2 * threadIdx.x; r < r1; r += 2 * BLOCK) {
    const uint64_t hv = ld_u64(h2 + r / 2);
    const uint32_t lo = f32_to_bf16(__uint_as_float((uint32_t)hv) + L.outc[r - r0]);
    const uint32_t hi = f32_to_bf16(__uint_as_float((uint32_t)(hv >> 32)) + L.outc[r + 1 - r0]);
    st_u32(xb + r / 2, lo | (hi << 16));
    if (out_hidden) gp(reinterpret_cast<uint32_t*>(out_hidden))[r / 2] = lo | (hi << 16);
  }
  stamp(a, cx, st, TR_DOWN_EPI);
  arrive(cx, S_OUT, st.k1, cx.nwg);
  stamp(a, cx, st, TR_DOWN_DONE);
  return true;
}

template <class SH>
__global__ void __launch_bounds__(BLOCK, 1) k_decode_gqa(KArgs a) {
  extern __shared__ float lds_raw[];
  Ctx cx;
  cx.budget = a.budget;
  cx.w = blockIdx.x;
  cx.nwg = gridDim.x;
  cx.ctr_xcd = wsp<uint32_t>(a, a.off.ctr_xcd);
  cx.ctr_glob = wsp<uint32_t>(a, a.off.ctr_glob);
  cx.ctr_grp = wsp<uint32_t>(a, a.off.ctr_grp);
  cx.ctr_att = wsp<uint32_t>(a, a.off.ctr_att);
  cx.status = wsp<uint32_t>(a, a.off.status);
  const DLayer* layers = wsp<DLayer>(a, a.off.layers);
  Lds L = carve(lds_raw, a.c);
  for (int t = 0; t < a.n_tokens; t++) {
    for (int li = 0; li < a.n_layers; li++) {
      cx.layer = a.layer0 + li;
      cx.token = t;
      Step st;
      st.Ly = layers + a.layer0 + li;
      st.idx = t * a.n_layers + li;
      st.k1 = a.step0 + (uint32_t)st.idx + 1u;
      st.first = (t == 0 && li == 0);
      st.in_hidden = st.first ? a.in_hidden : nullptr;
      st.pos = a.pos0 + t;
      const bool last = (t == a.n_tokens - 1) && (li == a.n_layers - 1);
      stamp(a, cx, st, TR_START);
      if (!stage_qkv_gqa<SH>(cx, a, st, L)) return;
      if (!attention_gqa<SH>(cx, a, st, L)) return;
      if (!stage_wo<SH>(cx, a, st, L)) return;
      if (!stage_ffn<SH>(cx, a, st, L)) return;
      if (!stage_down<SH>(cx, a, st, L, last ? a.out_hidden : nullptr)) return;
    }
  }
}

typedef void (*KernelFn)(KArgs);

// The compiled shapes: the tiny dense MHA layer (hidden 256, 4x64 heads, FFN 1024) and
// the GQA MoE layer (hidden 4096, 32 q / 8 kv heads x 128, 64 experts of width 1536).
using ShapeTinyDense = GqaShape<256, 4, 4, 64, 1024, false, false, 1, 2>;
using ShapeGqaMoe = GqaShape<4096, 32, 8, 128, 1536, false, true, 9, 33>;

template <class SH>
static bool matches(const pld_config* c) {
  return c->attn_kind == PLD_ATTN_GQA && c->hidden == SH::H && c->n_heads == SH::NH && c->n_kv_heads == SH::NKV &&
         c->head_dim == SH::HD && c->inter == SH::INTER && (c->wfmt == PLD_WFMT_FP8_BLOCK128) == SH::FP8 &&
         (c->ffn_kind == PLD_FFN_MOE) == SH::MOE;
}

static KernelFn pick_kernel(const pld_config* c) {
  if (matches<ShapeTinyDense>(c)) return k_decode_gqa<ShapeTinyDense>;
  if (matches<ShapeGqaMoe>(c)) return k_decode_gqa<ShapeGqaMoe>;
  return nullptr;
}

}  // namespace pld

// ====================================================================== host runtime
using namespace pld;

struct pld_handle {
  pld_config cfg;
  KCfg kc;
  WsOff off;
  int n_layers;
  uint8_t* ws;
  size_t ws_bytes;
  size_t lds_bytes;
  uint32_t steps;
  long long budget;
  int wallclock_khz;
  bool bad;
  bool coop;
  hipStream_t last_stream;
  KernelFn fn;
  int device;
  uint64_t* trace;
  int trace_steps;
};

namespace {

size_t al(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int device_cus(int* dev_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (dev_out) *dev_out = dev;
  return cus;
}

// Fills derived fields; returns PLD_OK or an error for unsupported shapes.
pld_status derive(const pld_config* c, int nwg, KCfg* k) {
  if (!c) return PLD_E_INVALID;
  memset(k, 0, sizeof(*k));
  k->attn = c->attn_kind; k->wfmt = c->wfmt; k->H = c->hidden; k->nh = c->n_heads; k->nkv = c->n_kv_heads;
  k->hd = c->head_dim; k->q_lora = c->q_lora; k->kv_lora = c->kv_lora; k->rope = c->rope_dim; k->nope = c->nope_dim;
  k->vdim = c->v_dim; k->ih = c->index_heads; k->idim = c->index_dim; k->itopk = c->index_topk; k->ffn = c->ffn_kind;
  k->inter = c->inter; k->E = c->n_experts; k->topk = c->top_k; k->nshared = c->n_shared; k->router = c->router_kind;
  k->max_seq = c->max_seq; k->vocab = c->vocab; k->eps = c->eps; k->nwg = nwg;
  if (c->hidden <= 0 || c->n_heads <= 0 || c->max_seq <= 0 || c->inter <= 0 || !(c->eps >= 0.0)) return PLD_E_INVALID;
  if (c->wfmt != PLD_WFMT_BF16 && c->wfmt != PLD_WFMT_FP8_BLOCK128) return PLD_E_UNSUPPORTED;
  if (nwg < NXCD || nwg % NXCD) return PLD_E_UNSUPPORTED;
  if (c->ffn_kind == PLD_FFN_DENSE) {
    k->slots = 1;
  } else if (c->ffn_kind == PLD_FFN_MOE) {
    if (c->n_experts < 8 || c->n_experts > nwg || c->n_experts > 512) return PLD_E_UNSUPPORTED;
    if (c->top_k < 1 || c->top_k > 16 || c->top_k > c->n_experts) return PLD_E_UNSUPPORTED;
    if (c->n_shared < 0 || c->n_shared > 2) return PLD_E_UNSUPPORTED;
    if (c->router_kind != PLD_ROUTER_SOFTMAX_TOPK && c->router_kind != PLD_ROUTER_SIGMOID_BIAS) return PLD_E_UNSUPPORTED;
    if (c->hidden % 8) return PLD_E_UNSUPPORTED;
    k->slots = c->top_k + c->n_shared;
    if (k->slots > MAX_SEGS) return PLD_E_UNSUPPORTED;
  } else {
    return PLD_E_UNSUPPORTED;
  }
  if (c->attn_kind == PLD_ATTN_GQA) {
    if (c->n_kv_heads <= 0 || c->n_heads % c->n_kv_heads) return PLD_E_UNSUPPORTED;
    k->G = c->n_heads / c->n_kv_heads;
    if (!pick_kernel(c)) return PLD_E_UNSUPPORTED;
    if (nwg % c->n_kv_heads) return PLD_E_UNSUPPORTED;
    k->cpg = nwg / c->n_kv_heads;
    k->chmax = (c->max_seq + k->cpg - 1) / k->cpg + 1;
    const int R = (c->n_heads + 2 * c->n_kv_heads) * c->head_dim;
    int act = std::max({c->hidden, c->n_heads * c->head_dim, k->slots * c->inter,
                        k->G * k->chmax + NWAVES * k->G * c->head_dim + 2 * k->G,
                        k->G * k->cpg * (c->head_dim + 2)});
    k->act_floats = (int)al(act, 64);
    k->stage_words = (int)al(c->hidden / 2 + 2, 64);
    int outb = std::max({R / nwg + 4, k->slots * (c->hidden / nwg + 4), 2 * ((k->slots * c->inter) / nwg + 2),
                         2 * (c->inter / nwg + 2) * std::max(1, c->n_shared), 4 * c->n_experts + 4});
    k->outb_floats = (int)al(outb, 64);
    if (lds_bytes_for(k->act_floats, k->stage_words, k->outb_floats) > 160 * 1024) return PLD_E_UNSUPPORTED;
  } else {
    return PLD_E_UNSUPPORTED;   // MLA path: not built yet
  }
  return PLD_OK;
}

WsOff layout(const KCfg& k, int n_layers) {
  WsOff o;
  size_t p = 0;
  o.ctr_xcd = p; p += al((size_t)NSTG * NXCD * CTR_STRIDE * 4);
  o.ctr_glob = p; p += al((size_t)NSTG * CTR_STRIDE * 4);
  const int ngrp = std::max(k.nkv, 1);
  o.ctr_grp = p; p += al((size_t)ngrp * CTR_STRIDE * 4);
  o.ctr_att = p; p += al((size_t)CTR_STRIDE * 4);
  o.status = p; p += al(64);
  o.xbuf = p; p += al((size_t)k.H * 4);
  o.q = p; p += al((size_t)std::max(k.nh * k.hd, 1) * 4);
  o.part = p; p += al((size_t)k.nh * k.cpg * (k.hd + 2) * 4);
  o.o = p; p += al((size_t)std::max(k.nh * k.hd, 1) * 4);
  o.h2 = p; p += al((size_t)k.H * 4);
  o.logits = p; p += al((size_t)std::max(k.E, 1) * 16);
  o.sel = p; p += al(64 * 4);
  o.gates = p; p += al(64 * 4);
  o.m = p; p += al((size_t)k.slots * k.inter * 4);
  o.a_dbg = p; p += al((size_t)k.H * 4);
  o.b_dbg = p; p += al((size_t)k.H * 4);
  o.rope = p; p += al((size_t)k.max_seq * std::max(k.hd, 2) * 4);
  o.layers = p; p += al((size_t)n_layers * sizeof(DLayer));
  o.total = p;
  return o;
}

DMat dmat(const pld_matrix& m, int rows, int cols, bool fp8) {
  DMat d;
  d.w = (const uint8_t*)m.data;
  d.s = fp8 ? m.scales : nullptr;
  d.rows = rows;
  d.cols = cols;
  d.sbk = (cols + 127) / 128;
  return d;
}

bool mat_ok(const pld_matrix& m, bool fp8) {
  return m.data && aligned16(m.data) && (!fp8 || (m.scales && aligned16(m.scales)));
}

}  // namespace

extern "C" {

const char* pld_status_string(pld_status s) {
  switch (s) {
    case PLD_OK: return "ok";
    case PLD_E_INVALID: return "invalid argument";
    case PLD_E_UNSUPPORTED: return "unsupported configuration";
    case PLD_E_CAPACITY: return "capacity exceeded (position or workspace)";
    case PLD_E_HIP: return "HIP runtime error";
    case PLD_E_DEVICE_TIMEOUT: return "device wait timed out";
    case PLD_E_STATE: return "handle needs decode_reset";
  }
  return "unknown status";
}

size_t pld_workspace_bytes(const pld_config* cfg, int32_t n_layers) {
  if (!cfg || n_layers < 1) return 0;
  const int nwg = device_cus(nullptr);
  if (nwg <= 0) return 0;
  KCfg k;
  if (derive(cfg, nwg, &k) != PLD_OK) return 0;
  return layout(k, n_layers).total;
}

pld_status decode_layer_init(const pld_config* cfg, int32_t n_layers, const pld_layer_weights* w,
                             const pld_kv_cache* kv, const pld_head_weights* head, void* workspace, size_t ws_bytes,
                             pld_handle** out) {
  if (!cfg || !w || !kv || !workspace || !out || n_layers < 1) return PLD_E_INVALID;
  *out = nullptr;
  if (!aligned16(workspace)) return PLD_E_INVALID;
  int dev = 0;
  const int nwg = device_cus(&dev);
  if (nwg <= 0) return PLD_E_HIP;
  KCfg k;
  pld_status st = derive(cfg, nwg, &k);
  if (st != PLD_OK) return st;
  if (cfg->vocab > 0 || head) return PLD_E_UNSUPPORTED;   // LM head: MLA stack only (not built yet)
  const WsOff off = layout(k, n_layers);
  if (ws_bytes < off.total) return PLD_E_CAPACITY;
  const bool fp8 = cfg->wfmt == PLD_WFMT_FP8_BLOCK128;
  const bool moe = cfg->ffn_kind == PLD_FFN_MOE;
  const int H = cfg->hidden;
  std::vector<DLayer> dl(n_layers);
  for (int l = 0; l < n_layers; l++) {
    const pld_layer_weights& L = w[l];
    DLayer& d = dl[l];
    memset(&d, 0, sizeof(d));
    if (!L.attn_norm || !L.ffn_norm || !aligned16(L.attn_norm) || !aligned16(L.ffn_norm)) return PLD_E_INVALID;
    d.attn_norm = L.attn_norm;
    d.ffn_norm = L.ffn_norm;
    const int hd = cfg->head_dim;
    if (!mat_ok(L.wq, fp8) || !mat_ok(L.wk, fp8) || !mat_ok(L.wv, fp8) || !mat_ok(L.wo, fp8)) return PLD_E_INVALID;
    d.wq = dmat(L.wq, cfg->n_heads * hd, H, fp8);
    d.wk = dmat(L.wk, cfg->n_kv_heads * hd, H, fp8);
    d.wv = dmat(L.wv, cfg->n_kv_heads * hd, H, fp8);
    d.wo = dmat(L.wo, H, cfg->n_heads * hd, fp8);
    if (!mat_ok(L.w_gate, fp8) || !mat_ok(L.w_up, fp8) || !mat_ok(L.w_down, fp8)) return PLD_E_INVALID;
    d.w_gate = dmat(L.w_gate, cfg->inter, H, fp8);
    d.w_up = dmat(L.w_up, cfg->inter, H, fp8);
    d.w_down = dmat(L.w_down, H, cfg->inter, fp8);
    const size_t wb = fp8 ? 1 : 2;
    d.gu_slot_bytes = (size_t)cfg->inter * H * wb;
    d.dn_slot_bytes = (size_t)H * cfg->inter * wb;
    d.gu_slot_scales = fp8 ? (size_t)((cfg->inter + 127) / 128) * ((H + 127) / 128) : 0;
    d.dn_slot_scales = fp8 ? (size_t)((H + 127) / 128) * ((cfg->inter + 127) / 128) : 0;
    if (moe) {
      if (!L.router || !aligned16(L.router)) return PLD_E_INVALID;
      d.router = (const uint16_t*)L.router;
      if (cfg->router_kind == PLD_ROUTER_SIGMOID_BIAS) {
        if (!L.router_bias) return PLD_E_INVALID;
        d.router_bias = L.router_bias;
      }
    }
    const pld_kv_cache& C = kv[l];
    if (!C.k || !C.v || !aligned16(C.k) || !aligned16(C.v)) return PLD_E_INVALID;
    d.kc = (uint16_t*)C.k;
    d.vc = (uint16_t*)C.v;
  }
  pld_handle* h = new (std::nothrow) pld_handle();
  if (!h) return PLD_E_INVALID;
  h->cfg = *cfg;
  h->kc = k;
  h->off = off;
  h->n_layers = n_layers;
  h->ws = (uint8_t*)workspace;
  h->ws_bytes = ws_bytes;
  h->lds_bytes = lds_bytes_for(k.act_floats, k.stage_words, k.outb_floats);
  h->steps = 0;
  h->bad = false;
  h->device = dev;
  h->last_stream = nullptr;
  h->trace = nullptr;
  h->trace_steps = 0;
  const char* coop = getenv("PLD_COOPERATIVE");
  h->coop = coop && atoi(coop) != 0;
  h->fn = pick_kernel(cfg);
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) khz = 100000;
  h->wallclock_khz = khz;
  h->budget = (long long)khz * 1000LL * 2;   // 2 s
  // RoPE table: (cos, sin) of pos * base^(-2i/d) for the interleaved pairs, fp64 -> fp32
  const int d = cfg->head_dim;
  std::vector<float> rope((size_t)cfg->max_seq * d);
  for (int p = 0; p < cfg->max_seq; p++)
    for (int i = 0; i < d / 2; i++) {
      const double ang = (double)p * std::pow(cfg->rope_base, -2.0 * i / d);
      rope[(size_t)p * d + 2 * i] = (float)std::cos(ang);
      rope[(size_t)p * d + 2 * i + 1] = (float)std::sin(ang);
    }
  bool ok = hipMemcpy(h->ws + off.rope, rope.data(), rope.size() * 4, hipMemcpyHostToDevice) == hipSuccess;
  ok = ok && hipMemcpy(h->ws + off.layers, dl.data(), dl.size() * sizeof(DLayer), hipMemcpyHostToDevice) == hipSuccess;
  ok = ok && hipMemset(h->ws, 0, off.xbuf) == hipSuccess;   // counters + status
  ok = ok && hipFuncSetAttribute((const void*)h->fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)h->lds_bytes) == hipSuccess;
  int per_cu = 0;
  ok = ok && hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)h->fn, BLOCK, h->lds_bytes) == hipSuccess;
  ok = ok && hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    delete h;
    return PLD_E_HIP;
  }
  if (per_cu < 1) {
    delete h;
    return PLD_E_UNSUPPORTED;
  }
  *out = h;
  return PLD_OK;
}

static pld_status launch(pld_handle* h, int layer0, int n_layers, int n_tokens, int pos0, const void* in_hidden,
                         void* out_hidden, hipStream_t s) {
  KArgs a;
  memset(&a, 0, sizeof(a));
  a.c = h->kc;
  a.ws = h->ws;
  a.off = h->off;
  a.n_layers = n_layers;
  a.n_tokens = n_tokens;
  a.pos0 = pos0;
  a.layer0 = layer0;
  a.step0 = h->steps;
  a.in_hidden = (const uint16_t*)in_hidden;
  a.out_hidden = (uint16_t*)out_hidden;
  a.budget = h->budget;
  a.trace = h->trace;
  a.trace_steps = h->trace_steps;
  hipError_t e;
  if (h->coop) {
    void* args[] = {&a};
    e = hipLaunchCooperativeKernel((const void*)h->fn, dim3(h->kc.nwg), dim3(BLOCK), args, (unsigned)h->lds_bytes, s);
  } else {
    void* args[] = {&a};
    e = hipLaunchKernel((const void*)h->fn, dim3(h->kc.nwg), dim3(BLOCK), args, h->lds_bytes, s);
  }
  if (e != hipSuccess) return PLD_E_HIP;
  h->steps += (uint32_t)(n_layers * n_tokens);
  h->last_stream = s;
  return PLD_OK;
}

pld_status decode_step(pld_handle* h, int32_t layer, const void* x_in, int32_t pos, void* x_out, void* stream) {
  if (!h || !x_in || !x_out || !aligned16(x_in) || !aligned16(x_out)) return PLD_E_INVALID;
  if (h->bad) return PLD_E_STATE;
  if (layer < 0 || layer >= h->n_layers) return PLD_E_INVALID;
  if (pos < 0 || pos >= h->cfg.max_seq) return PLD_E_CAPACITY;
  return launch(h, layer, 1, 1, pos, x_in, x_out, (hipStream_t)stream);
}

pld_status decode_layers_persistent(pld_handle* h, const pld_persistent_args* a, void* stream) {
  if (!h || !a) return PLD_E_INVALID;
  if (h->bad) return PLD_E_STATE;
  if (a->n_tokens < 1 || a->n_query != 1) return a->n_query > 1 ? PLD_E_UNSUPPORTED : PLD_E_INVALID;
  if (a->in_token >= 0) return PLD_E_UNSUPPORTED;   // embedding input needs the LM head path
  if (a->n_tokens != 1) return PLD_E_UNSUPPORTED;   // several tokens need the head (greedy loop)
  if (!a->in_hidden || !a->out_hidden || !aligned16(a->in_hidden) || !aligned16(a->out_hidden)) return PLD_E_INVALID;
  if (a->start_pos < 0 || a->start_pos + a->n_tokens > h->cfg.max_seq) return PLD_E_CAPACITY;
  return launch(h, 0, h->n_layers, a->n_tokens, a->start_pos, a->in_hidden, a->out_hidden, (hipStream_t)stream);
}

pld_status decode_poll_status(pld_handle* h, pld_device_status* out) {
  if (!h || !out) return PLD_E_INVALID;
  if (hipDeviceSynchronize() != hipSuccess) return PLD_E_HIP;
  int32_t st[8];
  if (hipMemcpy(st, h->ws + h->off.status, sizeof(st), hipMemcpyDeviceToHost) != hipSuccess) return PLD_E_HIP;
  memset(out, 0, sizeof(*out));
  out->code = st[ST_CODE];
  out->stage = st[ST_STAGE];
  out->layer = st[ST_LAYER];
  out->token = st[ST_TOKEN];
  out->wg = st[ST_WG];
  if (st[ST_CODE] != 0) {
    h->bad = true;
    return PLD_E_DEVICE_TIMEOUT;
  }
  return PLD_OK;
}

pld_status decode_reset(pld_handle* h) {
  if (!h) return PLD_E_INVALID;
  if (hipDeviceSynchronize() != hipSuccess) return PLD_E_HIP;
  if (hipMemset(h->ws, 0, h->off.xbuf) != hipSuccess) return PLD_E_HIP;
  if (hipDeviceSynchronize() != hipSuccess) return PLD_E_HIP;
  h->steps = 0;
  h->bad = false;
  return PLD_OK;
}

void decode_layer_destroy(pld_handle* h) { delete h; }

pld_status pld_debug_buffer(pld_handle* h, const char* name, void** ptr, size_t* bytes) {
  if (!h || !name || !ptr || !bytes) return PLD_E_INVALID;
  const KCfg& k = h->kc;
  struct E { const char* n; size_t off, sz; } tab[] = {
      {"a", h->off.a_dbg, (size_t)k.H * 4},
      {"q", h->off.q, (size_t)k.nh * k.hd * 4},
      {"o", h->off.o, (size_t)k.nh * k.hd * 4},
      {"h2", h->off.h2, (size_t)k.H * 4},
      {"b", h->off.b_dbg, (size_t)k.H * 4},
      {"logits", h->off.logits, (size_t)k.E * 16},
      {"sel", h->off.sel, (size_t)k.topk * 4},
      {"gates", h->off.gates, (size_t)k.topk * 4},
      {"m", h->off.m, (size_t)k.slots * k.inter * 4},
      {"x", h->off.xbuf, (size_t)k.H * 2},
  };
  for (auto& e : tab)
    if (!strcmp(e.n, name)) {
      *ptr = h->ws + e.off;
      *bytes = e.sz;
      return PLD_OK;
    }
  return PLD_E_INVALID;
}

pld_status pld_launch_shape(pld_handle* h, int32_t* n_wg, int32_t* block) {
  if (!h || !n_wg || !block) return PLD_E_INVALID;
  *n_wg = h->kc.nwg;
  *block = BLOCK;
  return PLD_OK;
}

pld_status pld_set_trace(pld_handle* h, void* buffer, size_t bytes) {
  if (!h) return PLD_E_INVALID;
  const size_t row = (size_t)h->kc.nwg * TR_SLOTS * sizeof(uint64_t);
  if (!buffer || bytes < row) {
    h->trace = nullptr;
    h->trace_steps = 0;
    return buffer ? PLD_E_CAPACITY : PLD_OK;
  }
  if (((uintptr_t)buffer & 7u) != 0) return PLD_E_INVALID;
  h->trace = (uint64_t*)buffer;
  h->trace_steps = (int)std::min(bytes / row, (size_t)1 << 20);
  return PLD_OK;
}

pld_status pld_set_watchdog_us(pld_handle* h, int64_t us) {
  if (!h || us <= 0) return PLD_E_INVALID;
  h->budget = (long long)((double)us * h->wallclock_khz / 1000.0);
  if (h->budget < 1) h->budget = 1;
  return PLD_OK;
}

}  // extern "C"
