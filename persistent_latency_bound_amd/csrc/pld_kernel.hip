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
#include <hip/hip_fp16.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <new>
#include <type_traits>
#include <vector>

#include "../../include/pld.h"
#include "pld_device.hpp"
#include "pld_math.hpp"

namespace pld {

// ------------------------------------------------------------------ shared structs
// Watchdog wait ids (pld_device_status.stage): which LL activation a workgroup waited for.
enum WaitId { W_X = 0, W_QKV = 1, W_KV = 2, W_PART = 3, W_O = 4, W_H2 = 5, W_RT = 6, W_M = 7, W_CQ = 8,
              W_QN = 9, W_QLAT = 10, W_OLAT = 11, W_AMAX = 12, W_IX = 13, W_ILIST = 14, W_ISEL = 15 };
enum { ST_CODE = 0, ST_STAGE = 1, ST_LAYER = 2, ST_TOKEN = 3, ST_WG = 4, ST_ABORT = 8 };
// device trace: wall-clock stamps per (step, workgroup)
enum TraceSlot {
  TR_START = 0, TR_X_READY, TR_QKV_DONE, TR_ATT_READY, TR_ATT_DONE, TR_O_READY, TR_WO_DONE, TR_H2_READY,
  TR_RT_READY, TR_FFN_DONE, TR_M_READY, TR_DOWN_DONE, TR_ATT_Q = 12, TR_ATT_SOFTMAX = 13, TR_ATT_PARTIAL = 14,
  TR_ATT_MERGED = 15, TR_TOPK = 16, TR_ROUTED_GEMV = 17, TR_M_STORED = 18, TR_DOWN_GEMV = 19, TR_DOWN_EPI = 20,
  TR_QKV_GEMV = 21, TR_SHARED_GEMV = 22, TR_ATT_PV = 23, TR_X_NORMED = 24, TR_MERGE_START = 25,
  TR_MERGE_COPIED = 26, TR_RT_LOGIT = 27, TR_ATT_DRAINED = 28, TR_ATT_SCORES = 30, TR_HEAD_READY = 32,
  TR_HEAD_GEMV = 33, TR_TOKEN = 34, TR_IDX_DONE = 35, TR_SEL_KEYS = 36, TR_SEL_PASSES = 37, TR_SEL_DONE = 38,
  TR_CQ_READY = 48, TR_Q_GEMV = 49,
  TR_WAIT = 50,   // not a stamp: total ticks the workgroup spent inside dependency waits (ll_fetch)
  TR_SLOTS = 56
};

struct KCfg {
  int attn, wfmt, H, nh, nkv, hd, q_lora, kv_lora, rope, nope, vdim, ih, idim, itopk, krank, cwidth;
  int ffn, inter, E, topk, nshared, router, max_seq, vocab;
  double eps;
  int slots;   // expert slots used per token (routed + shared), 1 for a dense FFN
  int G;       // q heads per kv head
  int cpg;     // attention chunks per kv head = workgroups per kv head
  int chmax;   // max tokens in one attention chunk
  int act_floats, stage_words, outb_floats;
  int nwg;
  int cpw;     // MLA: q_lat / o_lat outputs per workgroup (absorb, merge)
  int rdim;    // width of the RoPE table rows (head_dim for GQA, rope_dim for MLA)
  int vq;      // batched kernel: max rows (positions of a verify or sequences of a batch; 0: not set up)
  int vb;      // batch decode: sequences per layer cache (0: one sequence)
};

struct DLayer {
  const float *attn_norm, *ffn_norm, *q_norm, *kv_norm;
  DMat wq, wk, wv, wo, w_dq, w_uq, w_dkv, w_uk, w_uv, w_qi, w_w, w_ki;
  const uint16_t* router;
  const float* router_bias;
  DMat w_gate, w_up, w_down;
  size_t gu_slot_bytes, gu_slot_scales, dn_slot_bytes, dn_slot_scales;
  size_t gu_slot_cb, dn_slot_cb;   // LUT3 experts: codebook bytes per expert slot
  uint16_t *kc, *vc, *lat;
  uint8_t* icodes;
  float* iscales;
  DMat w_g, w_beta, w_adown, w_aup;   // KDA
  const float *conv_taps, *o_norm;
  float *kstate, *conv_ring;
};

// Workspace layout. The LL buffers (8-byte words: payload | epoch << 32) follow the
// status words; both are zeroed at init and by decode_reset.
struct WsOff {
  size_t status, x, q, kv, part, o, h2, logits, m, cqr, ckvr, qr, qlat, olat, amax, ixr, qi, ilist, isel, ll_end, sel,
      gates, spec, a_dbg, b_dbg, f_dbg, ikh, ikl, ilo, itok, kx, rope, layers, total;
  // batched verify (per-position copies of the LL buffers; vsel is a plain debug area)
  size_t vx, vcqr, vckv, vqn, vqr, vqlat, vpart, volat, vo, vh2, vss, vrp, vhn, vlog, vm, vfp, vamax, vsel, vf;
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
  // LM head (vocab > 0): greedy decode loop inside the launch
  const uint16_t* embed;   // bf16 [vocab][H]
  const float* fnorm;      // [H]
  DMat head;               // [vocab][H]
  float* out_logits;       // fp32 [n_tokens][vocab] or null
  int32_t* out_tokens;     // [n_tokens] or null
  int in_token;            // >= 0: first input is embed[in_token]
  int head_on;             // run the head after the last layer of every token
  const int32_t* drafts;   // verify: [n_tokens - 1] draft tokens fed to positions 1.., or null
  int32_t* out_accepted;   // verify: [1] accepted draft count, or null
  int hooks;               // test hooks (PLD_HOOK_*), 0 in normal use
  uint32_t hook_seed;
  double temperature;      // LM head: 0 = greedy argmax, > 0 = Gumbel-max sample of softmax(logits / T)
  uint64_t sample_seed;
  // batched kernel: rows per step; batch decode (bmode 1): per-sequence positions and input tokens
  int bmode, nrows;
  int32_t bpos[8], btok[8];
};

// ------------------------------------------------------------------ device context
struct Ctx {
  long long budget;   // watchdog budget of one wait, in wall-clock ticks
  int w, nwg;
  uint32_t* status;
  int layer, token;
  uint64_t* wacc;     // traced steps: LDS slot that accumulates the wait time (thread 0), else null
};

template <typename T>
__device__ __forceinline__ T* wsp(const KArgs& a, size_t off) {
  return reinterpret_cast<T*>(a.ws + off);
}

// Cold path: record the first expired wait and raise the abort flag.
__device__ __noinline__ void raise_timeout(uint32_t* status, int wait_id, int layer, int token, int w) {
  uint32_t expected = 0;
  if (__hip_atomic_compare_exchange_strong(gp(status + ST_CODE), &expected, (uint32_t)(int32_t)PLD_E_DEVICE_TIMEOUT,
                                           __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    st_u32(status + ST_STAGE, (uint32_t)wait_id);
    st_u32(status + ST_LAYER, (uint32_t)layer);
    st_u32(status + ST_TOKEN, (uint32_t)token);
    st_u32(status + ST_WG, (uint32_t)w);
  }
  st_u32(status + ST_ABORT, 1u);
}

// Test hook PLD_HOOK_DELAY: the workgroup waits a seeded pseudo-random time of up to 16 us
// (a hash of seed, workgroup, step and point) so that the stages of different workgroups
// run in another relative order. Every result is formed in a fixed order whatever the
// timing, so the outputs must not change. Bounded by the wall clock; all threads call it.
// The hash is Chris Wellons' "lowbias32" integer finalizer.
__device__ __noinline__ void test_delay(uint32_t seed, int w, int idx, int point) {
  uint32_t h = seed ^ ((uint32_t)w * 0x9E3779B9u) ^ ((uint32_t)idx * 0x85EBCA6Bu) ^ ((uint32_t)point * 0xC2B2AE35u);
  h ^= h >> 16; h *= 0x7feb352du; h ^= h >> 15; h *= 0x846ca68bu; h ^= h >> 16;
  const long long until = wall_clock64() + (long long)(h % 1600u);   // 100 MHz ticks
  while (wall_clock64() < until) __builtin_amdgcn_s_sleep(2);
}
#define PLD_TEST_DELAY(a, w, idx, point) \
  do { if ((a).hooks & PLD_HOOK_DELAY) test_delay((a).hook_seed, (w), (idx), (point)); } while (0)

// ------------------------------------------------------------------ LL handoff
// Every activation that crosses workgroups travels as LL words: one 8-byte atomic store
// carries a 32-bit payload in its low half and the epoch (step number + 1) in its high
// half, so a consumer that reads a word with the expected epoch has the payload too.
// There are no counters, no store drains and no atomics on the critical path: the
// producer stores and moves on; the consumer loads the words it needs and re-reads only
// those not yet published. Each LL buffer is written once per step, and every buffer's
// next write happens only after all its readers have moved past it (each consumer set
// depends on all producers of the following stage), so one buffer per activation is
// enough and a word can only hold the current epoch or an older one.
__device__ __forceinline__ uint64_t ll_word(uint32_t v, uint32_t ep) { return ((uint64_t)ep << 32) | v; }
__device__ __forceinline__ void ll_put(uint64_t* p, uint32_t v, uint32_t ep) { st_u64(p, ll_word(v, ep)); }
__device__ __forceinline__ void ll_put_f32(uint64_t* p, float v, uint32_t ep) { ll_put(p, __float_as_uint(v), ep); }

struct IdxLinear {
  __device__ __forceinline__ int operator()(int i) const { return i; }
};
// Where a fetched 32-bit payload goes: the word itself (default), or another placement.
struct StU32 {
  __device__ __forceinline__ void operator()(uint32_t* dst, int i, uint32_t v) const { dst[i] = v; }
};
// Word i of an activation vector into the layout apad<PAD> that gemv_list reads.
template <bool PAD>
struct StPad {
  __device__ __forceinline__ void operator()(uint32_t* dst, int i, uint32_t v) const { dst[apad<PAD>(i)] = v; }
};

// Reads the LL words src[idx(i)], i in [0, n), of epoch ep into dst[i] (LDS). PER loads
// per thread are issued together; words that are not yet published are re-read in a
// bounded loop (watchdog wait id wid). Every thread of the block must call; returns
// false (in every thread) on expiry or when another workgroup raised the abort flag.
template <int PER, typename Idx = IdxLinear, typename St = StU32>
__device__ __forceinline__ bool ll_fetch(Ctx& cx, uint32_t* dst, const uint64_t* src, int n, uint32_t ep, int wid,
                                         Idx idx = Idx{}, St store = St{}) {
  // one bit per load in the pending masks: a 64-bit mask past 32 loads (a shift by 32 or
  // more of a 32-bit value is undefined)
  static_assert(PER >= 1 && PER <= 64, "loads per thread and round");
  using Mask = typename std::conditional<(PER > 32), uint64_t, uint32_t>::type;
  int failed = 0;
  const int tid = tid_opaque();
  uint64_t t_in = 0;
  if (cx.wacc && tid == 0) t_in = wall_clock64();
  for (int base = 0; base < n; base += BLOCK * PER) {
    uint64_t v[PER];
#pragma unroll
    for (int j = 0; j < PER; j++) {
      const int i = base + j * BLOCK + tid;
      v[j] = i < n ? ld_u64_off(src, (uint32_t)idx(i) * 8u) : ll_word(0u, ep);
    }
    Mask pend = 0;
#pragma unroll
    for (int j = 0; j < PER; j++) pend |= (Mask)((uint32_t)(v[j] >> 32) != ep) << j;
    if (pend && !failed) {
      const long long deadline = wall_clock64() + cx.budget;
      int it = 0;
      while (pend) {
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int j = 0; j < PER; j++)
          if (pend >> j & 1u) v[j] = ld_u64_off(src, (uint32_t)idx(base + j * BLOCK + tid) * 8u);
        // (a mask of the words that arrived, built with shifts: constant masks ~(1 << j)
        // would be hoisted into registers that stay live across the whole kernel)
        Mask got = 0;
#pragma unroll
        for (int j = 0; j < PER; j++) got |= (Mask)((uint32_t)(v[j] >> 32) == ep) << j;
        pend &= ~got;
        if ((++it & 15) == 0 && pend) {
          if (ld_u32(cx.status + ST_ABORT)) { failed = 1; break; }
          if (wall_clock64() > deadline) { raise_timeout(cx.status, wid, cx.layer, cx.token, cx.w); failed = 1; break; }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < PER; j++) {
      const int i = base + j * BLOCK + tid;
      if (i < n) store(dst, i, (uint32_t)v[j]);
    }
  }
  const bool ok = !__syncthreads_or(failed);
  if (cx.wacc && tid == 0) *cx.wacc += wall_clock64() - t_in;
  return ok;
}
constexpr int per_for(int n) { return n <= BLOCK ? 1 : (n + BLOCK - 1) / BLOCK > 16 ? 16 : (n + BLOCK - 1) / BLOCK; }

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// The router's fp64 exp (pld_math.hpp) reads its constants from LDS (dk, written at kernel start).
__device__ __forceinline__ void exp_f64_init(double* dk) {
  if (tid_opaque() == 0) exp_f64_consts(dk);
}

// This thread's elements i = tid_opaque() + k*BLOCK of a length-N fp32 vector, held in
// registers. Small static vectors (norm weights) are loaded this way BEFORE a stage's
// weight prefetch is issued, so they sit at the front of the wave's in-order load queue
// instead of behind the weight loads.
template <int N>
struct RegVec {
  static constexpr int K = (N + BLOCK - 1) / BLOCK;
  float v[K];
  __device__ __forceinline__ void load(const float* p) {
    const PLD_GLOBAL float* g = gp(p);
#pragma unroll
    for (int k = 0; k < K; k++) {
      const int i = tid_opaque() + k * BLOCK;
      v[k] = (N % BLOCK == 0 || i < N) ? g[i] : 0.f;   // (a compile-time guard when it can be)
    }
  }
};
// In-place RMSNorm of the activation vector act (N elements, element i at act[apad<PAD>(i)]):
// act = fp32((act * r) * gamma), r = 1/sqrt(sum(act^2)/N + eps), statistics in fp64 (bf16
// and fp32 squares are exact in fp64); gamma in registers.
// (The thread's elements stay in registers between the two passes: re-reading them from
// LDS after writing earlier ones would serialize a full LDS round trip per element, since
// the compiler cannot tell the computed indices apart.)
template <int N, bool PAD>
__device__ __forceinline__ void rmsnorm_reg(float* act, const RegVec<N>& gam, double eps, double* red) {
  float xv[RegVec<N>::K];
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < RegVec<N>::K; k++) {
    const int i = tid_opaque() + k * BLOCK;
    xv[k] = (N % BLOCK == 0 || i < N) ? act[apad<PAD>(i)] : 0.f;
    ss += (double)xv[k] * (double)xv[k];
  }
  ss = block_sum(ss, red);
  const double r = 1.0 / sqrt(ss / (double)N + eps);
#pragma unroll
  for (int k = 0; k < RegVec<N>::K; k++) {
    const int i = tid_opaque() + k * BLOCK;
    if (N % BLOCK == 0 || i < N) act[apad<PAD>(i)] = (float)(((double)xv[k] * r) * (double)gam.v[k]);
  }
  __syncthreads();
}

// Weight loads in flight per lane for each GEMV stage (16-byte loads). Deep prefetch
// keeps HBM busy, but every load queued ahead of a latency-critical access in the same
// wave (an LL read of an activation) delays it, because a wave's loads return in order
// and the queue drains at the lane's share of HBM bandwidth. Chosen by measurement.
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

// LUT3 expert GEMVs: (row, 128-weight group) items in flight per lane (4 loads of 16 bytes each)
#ifndef PLD_LUT_ITEMS
#define PLD_LUT_ITEMS 2
#endif

constexpr int RT_SLOTS = 8;      // experts per lane in the router top-k: E <= 64 * RT_SLOTS
constexpr int RT_RANK_MAX = 64;  // up to this many experts the top-k counts ranks instead

// One (expert, slot, row range) piece of a gate/up GEMV list.
struct GuPiece { int expert, slot, j0, j1; };
constexpr int MAX_PIECES = MAX_SEGS / 2;

// ------------------------------------------------------------------ LDS layout
struct Lds {
  float* act;        // [act_floats]   activation vector / attention scratch / merge staging
  uint32_t* stage;   // [stage_words]  raw bf16-pair words of the incoming hidden state
  float* outb;       // [outb_floats]  GEMV row results
  float* outc;       // [outb_floats]
  float* xres;       // [outb_floats]  this workgroup's rows of the layer input (residual of W_o)
  float* h2res;      // [outb_floats]  this workgroup's rows of h2 (residual of the FFN)
  double* red;       // [16]
  int* isel;         // [32]
  float* fgate;      // [32]
  RowSeg* segs;      // [MAX_SEGS] GEMV segment list of the current stage
  uint64_t* tr;      // [TR_SLOTS] trace stamps of the current step (flushed at its end)
  double* dk;        // [16] fp64 constants of exp_f64 (kept in LDS, see there)
  GuPiece* pcs;      // [MAX_PIECES] gate/up pieces of the current list (LDS: a per-lane
                     // array indexed at run time would live in scratch memory)
};
__device__ __forceinline__ Lds carve(float* base, const KCfg& c) {
  Lds L;
  L.act = base;
  L.stage = reinterpret_cast<uint32_t*>(base + c.act_floats);
  L.outb = reinterpret_cast<float*>(L.stage + c.stage_words);
  L.outc = L.outb + c.outb_floats;
  L.xres = L.outc + c.outb_floats;
  L.h2res = L.xres + c.outb_floats;
  L.red = reinterpret_cast<double*>(L.h2res + c.outb_floats);
  L.isel = reinterpret_cast<int*>(L.red + 16);
  L.fgate = reinterpret_cast<float*>(L.isel + 32);
  L.segs = reinterpret_cast<RowSeg*>(L.fgate + 32);
  L.tr = reinterpret_cast<uint64_t*>(L.segs + MAX_SEGS);
  L.dk = reinterpret_cast<double*>(L.tr + TR_SLOTS);
  L.pcs = reinterpret_cast<GuPiece*>(L.dk + 16);
  return L;
}
__host__ __device__ inline size_t lds_bytes_for(int act_floats, int stage_words, int outb_floats) {
  return (size_t)4 * (act_floats + stage_words + 4 * outb_floats) + 8 * 16 + 4 * 32 + 4 * 32 +
         sizeof(RowSeg) * MAX_SEGS + 8 * TR_SLOTS + 8 * 16 + sizeof(GuPiece) * MAX_PIECES;
}

// Publishes a segment list to the workgroup (the previous list must be out of use).
__device__ __forceinline__ void seg_begin() { __syncthreads(); }
__device__ __forceinline__ void seg_set(Lds& L, int i, const uint8_t* w, const float* sc, int n, int srow, int act_off,
                                        float alpha) {
  if (tid_opaque() == 0) {
    RowSeg& S = L.segs[i];
    // alpha as a per-call value: a constant alpha would be paired with act_off into one
    // 64-bit constant, hoisted to kernel entry and kept live (and spilled) across stages
    asm volatile("" : "+v"(alpha));
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
  static constexpr bool LUTX = false;   // expert matrices in the weight format of the layer
  static_assert(H % 2 == 0 && ODIM % 2 == 0, "hidden sizes must be even");
};

// Per-(token, layer) state of one workgroup.
struct Step {
  const DLayer* Ly;
  const uint16_t* in_hidden;   // caller's bf16 input for the first step of the launch, else null
  uint32_t k1;                 // step number + 1 (LL epoch of this step)
  bool first;                  // first step of the launch
  int pos;
  int idx;                     // step index within the launch (trace row)
  uint64_t* tr;                // LDS stamps of this step (thread 0)
  const uint16_t* emb_row;     // embedding row that is this step's input (first layer of a token), or null
};

// Device trace: thread 0 keeps the step's stamps in LDS (a global store here would be
// waited for by the next in-order load wait of wave 0 and distort what it measures);
// trace_flush writes them out once per step.
__device__ __forceinline__ void stamp(const KArgs& a, const Ctx& cx, const Step& st, int slot) {
  if (a.trace && st.idx < a.trace_steps && tid_opaque() == 0) st.tr[slot] = wall_clock64();
}
__device__ __forceinline__ void trace_flush(const KArgs& a, const Ctx& cx, const Step& st) {
  if (a.trace && st.idx < a.trace_steps && tid_opaque() == 0) {
    PLD_GLOBAL uint64_t* dst = gp(a.trace) + ((size_t)st.idx * cx.nwg + cx.w) * TR_SLOTS;
    for (int i = 0; i < TR_SLOTS; i++) {
      dst[i] = st.tr[i];
      st.tr[i] = 0;
    }
  }
}

// Rows [r0, r1) of an H-row stage for this workgroup, split in pairs (the hidden state
// moves between workgroups as packed bf16 pairs).
__device__ __forceinline__ void hrows(int H, int nwg, int w, int* r0, int* r1) {
  *r0 = 2 * split_at(H / 2, nwg, w);
  *r1 = 2 * split_at(H / 2, nwg, w + 1);
}

// The layer input of a step: an embedding row (first layer of a token with a head), the
// caller's bf16 vector (first step of the launch) or the previous step's output (LL
// words of bf16 pairs, previous epoch); expanded to fp32 in L.act (layout apad<PAD>),
// this workgroup's residual rows [h0, h1) kept in L.xres, then RMSNorm in place.
template <int H, bool PAD>
__device__ __forceinline__ bool layer_input(Ctx& cx, const KArgs& a, const Step& st, Lds& L, const RegVec<H>& gam,
                                            int h0, int h1) {
  if (st.emb_row || st.first) {
    const PLD_GLOBAL uint32_t* src = gp(reinterpret_cast<const uint32_t*>(st.emb_row ? st.emb_row : st.in_hidden));
    for (int i = tid_opaque(); i < H / 2; i += BLOCK) L.stage[i] = src[i];
    __syncthreads();
  } else if (!ll_fetch<per_for(H / 2)>(cx, L.stage, wsp<uint64_t>(a, a.off.x), H / 2, st.k1 - 1u, W_X)) {
    return false;
  }
  stamp(a, cx, st, TR_X_READY);
#pragma unroll
  for (int k = 0; k < (H / 2 + BLOCK - 1) / BLOCK; k++) {
    const int i = tid_opaque() + k * BLOCK;
    if ((H / 2) % BLOCK == 0 || i < H / 2) {
      const uint32_t v = L.stage[i];
      *reinterpret_cast<float2*>(L.act + apad<PAD>(2 * i)) = make_float2(bf_lo(v), bf_hi(v));
    }
  }
  __syncthreads();
  for (int r = h0 + tid_opaque(); r < h1; r += BLOCK) L.xres[r - h0] = L.act[apad<PAD>(r)];
  rmsnorm_reg<H, PAD>(L.act, gam, a.c.eps, L.red);
  stamp(a, cx, st, TR_X_NORMED);
  if (cx.w == 0)
    for (int i = tid_opaque(); i < H; i += BLOCK) st_f32(wsp<float>(a, a.off.a_dbg) + i, L.act[apad<PAD>(i)]);
  return true;
}

// ------------------------------------------------------------------ stage: RMSNorm + QKV + RoPE + cache append
template <class SH>
__device__ __forceinline__ bool stage_qkv_gqa(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  constexpr int HD = SH::HD;
  const int w = cx.w, nwg = cx.nwg, pos = st.pos;
  const uint32_t k1 = st.k1;
  constexpr int qR = SH::NH * HD, kR = SH::NKV * HD, R = qR + 2 * kR;
  constexpr int P = R / 2;
  const int r0 = 2 * split_at(P, nwg, w), r1 = 2 * split_at(P, nwg, w + 1);
  int h0, h1;
  hrows(SH::H, nwg, w, &h0, &h1);
  RegVec<SH::H> gam;
  gam.load(Ly.attn_norm);
  // RoPE (cos, sin) of this thread's first output pair, loaded before the GEMV: after it,
  // a global load would queue behind the GEMV's trailing weight loads
  const PLD_GLOBAL float* rope = gp(wsp<float>(a, a.off.rope)) + (size_t)pos * HD;   // (cos, sin) pairs
  float rcs = 1.f, rsn = 0.f;
  {
    const int r = 2 * (r0 / 2 + tid_opaque());
    if (r < r1 && r < qR + kR) {
      const int d = (r < qR ? r : r - qR) % HD;
      rcs = rope[d];
      rsn = rope[d + 1];
    }
  }
  bool pending = true;   // the input read + RMSNorm has not run yet
  auto pre_x = [&]() -> bool {
    if (!pending) return true;
    pending = false;
    return layer_input<SH::H, SH::FP8>(cx, a, st, L, gam, h0, h1);
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
  // RoPE on q and k; q -> LL (fp32); k, v -> cache row (bf16) and LL (bf16 pairs) for
  // this step's attention
  uint64_t* qll = wsp<uint64_t>(a, a.off.q);
  uint64_t* kvll = wsp<uint64_t>(a, a.off.kv);   // [k: NKV*HD/2 | v: NKV*HD/2] bf16-pair words
  for (int p = r0 / 2 + tid_opaque(); p < r1 / 2; p += BLOCK) {
    const int r = 2 * p;
    float v0 = L.outb[r - r0], v1 = L.outb[r + 1 - r0];
    if (r < qR + kR) {
      const int d = (r < qR ? r : r - qR) % HD;
      const bool first = p == r0 / 2 + tid_opaque();
      const float cs = first ? rcs : rope[d], sn = first ? rsn : rope[d + 1];
      const float x0 = v0 * cs - v1 * sn, x1 = v0 * sn + v1 * cs;
      v0 = x0;
      v1 = x1;
    }
    if (r < qR) {
      ll_put_f32(qll + r, v0, k1);
      ll_put_f32(qll + r + 1, v1, k1);
    } else {
      const bool isk = r < qR + kR;
      const int rr = isk ? r - qR : r - qR - kR;
      const int head = rr / HD, d = rr % HD;
      const uint32_t pair = f32_to_bf16(v0) | (f32_to_bf16(v1) << 16);
      uint16_t* dst = (isk ? Ly.kc : Ly.vc) + ((size_t)head * c.max_seq + pos) * HD + d;
      st_u32(reinterpret_cast<uint32_t*>(dst), pair);
      ll_put(kvll + (isk ? 0 : kR / 2) + rr / 2, pair, k1);
    }
  }
  stamp(a, cx, st, TR_QKV_DONE);
  return true;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ attention (GQA)
// One workgroup = one (kv head g, token chunk) pair. Scores for the G query heads of
// the group, chunk-local softmax, P.V, then a partial (m, l, acc[HD]) per head; then
// each workgroup of the group merges its own slice of the group's outputs.
//  * scores of the static history rows on the matrix cores (mfma 16x16x32 bf16): a wave
//    takes 16 rows per product, lane l holding 16 bytes of row l % 16 (its 16-byte chunks
//    l / 16 + 4 ks), exactly the B operand; q (fp32) enters as a bf16 high and low part
//    (two products), so the scores keep fp32-level q; the rows written inside the launch
//    take the vector path (16-byte K loads, HD/8 lanes per row, DPP row sums);
//  * P.V: each wave owns a contiguous token range and each lane HD/64 dims, so the sum
//    over tokens needs no lane exchange, only one cross-wave pass through LDS;
//  * the static history rows of the first batch (K and V) are issued before q is read;
//    the row of this step comes from the LL words of the QKV stage, and rows written by
//    earlier steps of this launch are read with coherent loads.
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
  // wave index as a provably uniform value: per-wave bounds then branch on scalars
  const int lane = tid_opaque() & 63, wave = __builtin_amdgcn_readfirstlane(tid_opaque() >> 6);
  const int dl = lane % LPT, tl = lane / LPT;
  const int cpg = c.cpg;
  const int g = cx.w / cpg, ch = cx.w % cpg;
  if (g >= SH::NKV) return true;   // workgroups past the last group have no attention work
  const int pos = st.pos;
  const int T = pos + 1;
  const int t0 = split_at(T, cpg, ch), t1 = split_at(T, cpg, ch + 1), n = t1 - t0;
  const int tw = (n + NWAVES - 1) / NWAVES;             // P.V tokens per wave
  const int pv0 = min(n, wave * tw), pv1 = min(n, pv0 + tw);
  const uint16_t* kbase = Ly.kc + (size_t)g * c.max_seq * HD + dl * 8;
  const uint16_t* vbase = Ly.vc + (size_t)g * c.max_seq * HD + lane * DPL;
  const int fresh = a.pos0;   // rows >= fresh were written inside this launch
  // LDS: q of the group [G][HD], the new k and v rows [HD/2 + HD/2 words], scores, ...
  float* qs = L.act;
  uint32_t* kvn = reinterpret_cast<uint32_t*>(L.act + G * HD);
  float* sc = L.act + G * HD + HD;                 // [G][chmax]
  float* red2 = sc + G * c.chmax;                  // [NWAVES][G][HD]
  float* ml = red2 + NWAVES * G * HD;              // [2G]
  // [2][G][HD] bf16: scaled q, high and low parts (16-byte aligned for the operand reads)
  uint16_t* qhl = reinterpret_cast<uint16_t*>(L.act + (((int)(ml + 2 * G - L.act) + 3) & ~3));
  // Rows [0, nst) of the chunk are static history (written before this launch) and are
  // streamed with plain loads; rows [nst, n) were written inside this launch (row pos by
  // this step) and are handled by a separate short pass. Static loads are unconditional:
  // an index past the static rows is clamped to the last one (its result is unused), so
  // no load sits under a condition and the in-order load waits stay exact.
  const int nst = max(0, min(n, fresh - t0));
  auto srow = [&](int t) -> size_t { return (size_t)(nst > 0 ? t0 + min(t, nst - 1) : 0); };
  // V element(s) of this lane for token t (DPL bf16 values packed in a word)
  auto v_static = [&](int t) -> uint32_t {
    const uint16_t* p = vbase + srow(t) * HD;
    if constexpr (DPL == 2) return *(const PLD_GLOBAL uint32_t*)(p);
    else return (uint32_t)(*(const PLD_GLOBAL uint16_t*)(p));
  };
  // fresh rows: row pos from the LL copy in LDS, earlier rows of this launch coherently
  auto k_fresh = [&](int t) -> uint4 {
    if (t0 + t == pos) {
      const uint32_t* q = kvn + dl * 4;
      return make_uint4(q[0], q[1], q[2], q[3]);
    }
    const uint64_t* q = reinterpret_cast<const uint64_t*>(kbase + (size_t)(t0 + t) * HD);
    const uint64_t x = ld_u64(q), y = ld_u64(q + 1);
    return make_uint4((uint32_t)x, (uint32_t)(x >> 32), (uint32_t)y, (uint32_t)(y >> 32));
  };
  auto v_fresh = [&](int t) -> uint32_t {
    if (t0 + t == pos) {
      if constexpr (DPL == 2) return kvn[HD / 2 + lane];
      else return (kvn[HD / 2 + lane / 2] >> (16 * (lane & 1))) & 0xffffu;
    }
    const uint16_t* p = vbase + (size_t)(t0 + t) * HD;
    if constexpr (DPL == 2) return ld_u32(reinterpret_cast<const uint32_t*>(p));
    else {
      const uint32_t w2 = ld_u32(reinterpret_cast<const uint32_t*>(p - (lane & 1)));
      return (lane & 1) ? (w2 >> 16) : (w2 & 0xffffu);
    }
  };
  const int pvs = min(pv1, max(pv0, nst));   // this wave's static P.V rows are [pv0, pvs)
  // static K rows in the matrix-core layout: group pass gp holds rows gp*GT + 16*wave + (lane & 15)
  constexpr int KS = HD / 32;                        // k-steps of 32 dims
  constexpr int GT = NWAVES * 16;                    // rows per group pass
  constexpr int NGR = NB * PASS / GT > 0 ? NB * PASS / GT : 1;   // group passes in registers
  static_assert(HD % 32 == 0 && G <= 16, "matrix-core scores");
  const uint16_t* kmat = Ly.kc + (size_t)g * c.max_seq * HD + ((lane >> 4) * 8);
  auto k_mf = [&](int t, int ks) -> uint4 { return ld_g16(kmat + srow(t) * HD + ks * 32); };
  auto mrow = [&](int tb0, int gp) { return tb0 + gp * GT + wave * 16 + (lane & 15); };
  uint4 kb[NGR][KS];
  uint32_t vb[NV];
#pragma unroll
  for (int gp = 0; gp < NGR; gp++)
#pragma unroll
    for (int ks = 0; ks < KS; ks++) kb[gp][ks] = k_mf(mrow(0, gp), ks);
#pragma unroll
  for (int b = 0; b < NV; b++) vb[b] = v_static(pv0 + b);
  // q of the group and, for the chunk that holds position pos, the new k/v row: one fetch
  // (both come from the QKV stage; kvn follows qs in LDS)
  {
    constexpr int kR2 = SH::NKV * HD / 2;
    const uint32_t qw = (uint32_t)(a.off.q / 8) + (uint32_t)(g * G * HD), kvw = (uint32_t)(a.off.kv / 8);
    auto idx = [=](int i) -> int {
      if (i < G * HD) return (int)qw + i;
      const int j = i - G * HD;
      return (int)kvw + (j < HD / 2 ? g * (HD / 2) + j : kR2 + g * (HD / 2) + (j - HD / 2));
    };
    const int nw = G * HD + ((t0 <= pos && pos < t1) ? HD : 0);
    if (!ll_fetch<per_for(G * HD + HD)>(cx, reinterpret_cast<uint32_t*>(qs), reinterpret_cast<const uint64_t*>(a.ws),
                                        nw, k1, W_QKV, idx))
      return false;
  }
  stamp(a, cx, st, TR_ATT_READY);
  const float scale = 1.0f / sqrtf((float)HD);
  float qr[G][8];
#pragma unroll
  for (int h = 0; h < G; h++)
#pragma unroll
    for (int j = 0; j < 8; j++) qr[h][j] = qs[h * HD + dl * 8 + j] * scale;
  // scaled q as bf16 high + low parts for the matrix cores (the pair carries 16 bits)
  for (int i = tid_opaque(); i < G * HD; i += BLOCK) {
    const float v = qs[i] * scale;
    const uint32_t hb = f32_to_bf16(v);
    qhl[i] = (uint16_t)hb;
    qhl[G * HD + i] = (uint16_t)f32_to_bf16(v - __uint_as_float(hb << 16));
  }
  __syncthreads();
  stamp(a, cx, st, TR_ATT_Q);
  auto score = [&](int t, const uint4& kv, int lim) {
    const float kf[8] = {bf_lo(kv.x), bf_hi(kv.x), bf_lo(kv.y), bf_hi(kv.y),
                         bf_lo(kv.z), bf_hi(kv.z), bf_lo(kv.w), bf_hi(kv.w)};
#pragma unroll
    for (int h = 0; h < G; h++) {
      float sh = 0.f;
#pragma unroll
      for (int j = 0; j < 8; j++) sh = fmaf(qr[h][j], kf[j], sh);
      sh = dpp_sum<LPT>(sh);
      if (dl == LPT - 1 && t < lim) sc[h * c.chmax + t] = sh;
    }
  };
  // ---- pass 1: scores of the static rows on the matrix cores (next group issued as each
  // register set frees up; rows past nst are computed on clamped data and not stored)
  {
    const int qm = lane & 15;   // A operand row (head); rows >= G are zero
    auto qop = [&](int part, int ks) -> bf16x8_t {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (qm < G) v = *reinterpret_cast<const uint4*>(qhl + part * G * HD + qm * HD + ks * 32 + (lane >> 4) * 8);
      return __builtin_bit_cast(bf16x8_t, v);
    };
    for (int tb0 = 0; tb0 < nst; tb0 += NGR * GT) {
#pragma unroll
      for (int gp = 0; gp < NGR; gp++) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
          const bf16x8_t kv = __builtin_bit_cast(bf16x8_t, kb[gp][ks]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qop(0, ks), kv, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qop(1, ks), kv, acc, 0, 0, 0);
        }
        // lane l holds heads 4 (l / 16) + i of row (l % 16)
        const int t = mrow(tb0, gp);
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int h = 4 * (lane >> 4) + i;
          if (h < G && t < nst) sc[h * c.chmax + t] = acc[i];
        }
      }
      if (tb0 + NGR * GT < nst) {
#pragma unroll
        for (int gp = 0; gp < NGR; gp++)
#pragma unroll
          for (int ks = 0; ks < KS; ks++) kb[gp][ks] = k_mf(mrow(tb0 + NGR * GT, gp), ks);
      }
    }
  }
  // ---- scores of the fresh rows
  for (int t = nst + wave * TPW + tl; t - tl < n; t += PASS) {
    const uint4 kv = t < n ? k_fresh(t) : make_uint4(0u, 0u, 0u, 0u);
    score(t, kv, n);
  }
  stamp(a, cx, st, TR_ATT_SCORES);
  __syncthreads();
  for (int h = wave; h < G; h += NWAVES) {
    float m = -INFINITY;
    for (int t = lane; t < n; t += 64) m = fmaxf(m, sc[h * c.chmax + t]);
    m = wave_max_dpp(m);
    float l = 0.f;
    for (int t = lane; t < n; t += 64) {
      const float p = __expf(sc[h * c.chmax + t] - m);
      sc[h * c.chmax + t] = p;
      l += p;
    }
    l = wave_sum_dpp(l);
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
  // p of row t, or 0 past `lim` (a select, not a branch: the reads stay in flight
  // together; sc has slack past the last row of every head, inside the LDS carve)
  auto pv = [&](int t, uint32_t vv, int lim) {
    const float v0 = bf_lo(vv);
    const float v1 = DPL == 2 ? bf_hi(vv) : 0.f;
#pragma unroll
    for (int h = 0; h < G; h++) {
      const float raw = sc[h * c.chmax + t];   // t < tb + NV: inside sc + red2 for every head
      const float p = t < lim ? raw : 0.f;
      acc[h][0] = fmaf(p, v0, acc[h][0]);
      if constexpr (DPL == 2) acc[h][1] = fmaf(p, v1, acc[h][1]);
    }
  };
  for (int tb = pv0; tb < pvs; tb += NV) {
#pragma unroll
    for (int b = 0; b < NV; b++) {
      pv(tb + b, vb[b], pvs);
      // at most 8 rows of LDS reads in flight: bounds register pressure (no spills)
      if ((b & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
    if (tb + NV < pvs) {
#pragma unroll
      for (int b = 0; b < NV; b++) vb[b] = v_static(tb + NV + b);
    }
  }
  for (int t = pvs; t < pv1; t++) pv(t, v_fresh(t), pv1);
#pragma unroll
  for (int h = 0; h < G; h++)
#pragma unroll
    for (int e = 0; e < DPL; e++) red2[(wave * G + h) * HD + lane * DPL + e] = acc[h][e];
  stamp(a, cx, st, TR_ATT_PV);
  // The cache rows this workgroup appended (QKV stage) must be visible before its next
  // publication: later steps of the launch read them with coherent loads.
  vm_wait();
  __syncthreads();
  stamp(a, cx, st, TR_ATT_DRAINED);
  // partial of head h for this chunk: LL words [m, l, acc[0..HD)] at ((g*G + h)*cpg + ch)*(HD+2)
  uint64_t* pll = wsp<uint64_t>(a, a.off.part);
  for (int i = tid_opaque(); i < G * HD; i += BLOCK) {
    const int h = i / HD, d = i % HD;
    float s = 0.f;
#pragma unroll
    for (int wv = 0; wv < NWAVES; wv++) s += red2[(wv * G + h) * HD + d];
    ll_put_f32(pll + ((size_t)(g * G + h) * cpg + ch) * (HD + 2) + 2 + d, s, k1);
  }
  if (tid_opaque() < 2 * G) {
    const int h = tid_opaque() >> 1;
    ll_put_f32(pll + ((size_t)(g * G + h) * cpg + ch) * (HD + 2) + (tid_opaque() & 1), ml[tid_opaque()], k1);
  }
  stamp(a, cx, st, TR_ATT_PARTIAL);
  // Distributed merge: workgroup ch of the group merges dims [d0, d1) of the group's G*HD
  // outputs (flash-decoding rescale: o = sum_c e^(m_c - M) acc_c / sum_c e^(m_c - M) l_c
  // over the chunks with l_c > 0), reading the cpg partials' LL words it needs.
  {
    const int d0 = split_at(G * HD, cpg, ch), d1 = split_at(G * HD, cpg, ch + 1), nd = d1 - d0;
    const int h0 = d0 / HD, nh2 = nd > 0 ? (d1 - 1) / HD - h0 + 1 : 0;
    const uint64_t* pg = pll + (size_t)g * G * cpg * (HD + 2);
    // word i < cpg*nd: acc of (chunk i / nd, dim d0 + i % nd); then (m, l) of head h0 + hh, chunk cc
    const int nacc = cpg * nd;
    auto pidx = [=](int i) -> int {
      if (i < nacc) {
        const int cc = i / nd, d = d0 + i % nd;
        return ((d / HD) * cpg + cc) * (HD + 2) + 2 + d % HD;
      }
      const int j = i - nacc, hh = j / (2 * cpg), r = j % (2 * cpg);
      return ((h0 + hh) * cpg + (r >> 1)) * (HD + 2) + (r & 1);
    };
    float* accs = L.act;              // [cpg][nd]
    float* mls = L.act + nacc;        // [nh2][cpg][2]
    __syncthreads();                  // L.act (scores) is free again
    stamp(a, cx, st, TR_MERGE_START);
    if (!ll_fetch<2>(cx, reinterpret_cast<uint32_t*>(L.act), pg, nacc + 2 * cpg * nh2, k1, W_PART, pidx)) return false;
    stamp(a, cx, st, TR_MERGE_COPIED);
    // wave hh computes the chunk weights of head h0 + hh: f_c = e^(m_c - M) for l_c > 0
    // (else 0) with M the max over those chunks, and Ls = sum_c f_c l_c
    float* fw = mls + 2 * cpg * nh2;   // [nh2][cpg]
    float* lsum = fw + cpg * nh2;      // [nh2]
    if (wave < nh2) {
      const float* ml2 = mls + 2 * cpg * wave;
      float M = -INFINITY;
      for (int cc = lane; cc < cpg; cc += 64)
        if (ml2[2 * cc + 1] > 0.f) M = fmaxf(M, ml2[2 * cc]);
      M = wave_max_dpp(M);
      float ls = 0.f;
      for (int cc = lane; cc < cpg; cc += 64) {
        const float l = ml2[2 * cc + 1];
        const float f = l > 0.f ? __expf(ml2[2 * cc] - M) : 0.f;
        fw[wave * cpg + cc] = f;
        ls += f * l;
      }
      ls = wave_sum_dpp(ls);
      if (lane == 0) lsum[wave] = ls;
    }
    __syncthreads();
    uint64_t* oll = wsp<uint64_t>(a, a.off.o) + (size_t)g * G * HD;
    for (int j = tid_opaque(); j < nd; j += BLOCK) {
      const int d = d0 + j, hh = d / HD - h0;
      const float* f = fw + hh * cpg;
      float o4[4] = {0.f, 0.f, 0.f, 0.f};   // four independent chains, added in a fixed order
      int cc = 0;
      for (; cc + 4 <= cpg; cc += 4) {
#pragma unroll
        for (int u = 0; u < 4; u++) o4[u] = fmaf(f[cc + u], accs[(cc + u) * nd + j], o4[u]);
      }
      for (; cc < cpg; cc++) o4[0] = fmaf(f[cc], accs[cc * nd + j], o4[0]);
      const float o = (o4[0] + o4[1]) + (o4[2] + o4[3]);
      ll_put_f32(oll + d, o / lsum[hh], k1);
    }
  }
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
    if (!ll_fetch<per_for(SH::ODIM)>(cx, reinterpret_cast<uint32_t*>(L.act), wsp<uint64_t>(a, a.off.o), SH::ODIM,
                                     st.k1, W_O, IdxLinear{}, StPad<SH::FP8>{}))
      return false;
    stamp(a, cx, st, TR_O_READY);
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
  // h2 = x + W_o o: LL words for every consumer, and this workgroup's rows kept in LDS
  // for the FFN residual (the down stage owns the same rows)
  uint64_t* h2ll = wsp<uint64_t>(a, a.off.h2);
  for (int r = r0 + tid_opaque(); r < r1; r += BLOCK) {
    const float v = L.xres[r - r0] + L.outb[r - r0];
    L.h2res[r - r0] = v;
    ll_put_f32(h2ll + r, v, st.k1);
  }
  stamp(a, cx, st, TR_WO_DONE);
  return true;
}

// ------------------------------------------------------------------ stage: FFN gate/up (+ router)
// Gate/up rows of several (expert, slot, row range) pieces as one GEMV list, then
// m[slot][j] = silu(gate_j . b) * (up_j . b), published as LL words. Each piece
// contributes a gate segment and an up segment; results come back in list order.
template <class SH, int INFL, typename Pre>
__device__ __forceinline__ bool gate_up_list(const KArgs& a, const Step& st, Lds& L, int np, Pre&& pre) {
  const GuPiece* pc = L.pcs;   // written by thread 0 before the call, published by seg_begin
  const DLayer Ly = *gp(st.Ly);
  constexpr size_t RB = SH::LUTX ? (size_t)SH::H * 3 / 8 : (size_t)SH::H * (SH::FP8 ? 1 : 2);
  seg_begin();
  for (int p = 0; p < np; p++) {
    const size_t bo = (size_t)pc[p].expert * Ly.gu_slot_bytes + (size_t)pc[p].j0 * RB;
    const float* sg;
    const float* su;
    if constexpr (SH::LUTX) {   // the slot's codebooks (bytes)
      sg = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(Ly.w_gate.s) + pc[p].expert * Ly.gu_slot_cb);
      su = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(Ly.w_up.s) + pc[p].expert * Ly.gu_slot_cb);
    } else {
      sg = SH::FP8 ? Ly.w_gate.s + (size_t)pc[p].expert * Ly.gu_slot_scales : nullptr;
      su = SH::FP8 ? Ly.w_up.s + (size_t)pc[p].expert * Ly.gu_slot_scales : nullptr;
    }
    seg_set(L, 2 * p, Ly.w_gate.w + bo, sg, pc[p].j1 - pc[p].j0, pc[p].j0, 0, 1.f);
    seg_set(L, 2 * p + 1, Ly.w_up.w + bo, su, pc[p].j1 - pc[p].j0, pc[p].j0, 0, 1.f);
  }
  seg_end();
  if constexpr (SH::LUTX) {
    if (!gemv_list_lut<SH::H, PLD_LUT_ITEMS>(L.segs, 2 * np, L.act, L.outb, OUT_STORE, pre)) return false;
  } else {
    if (!gemv_list<SH::FP8, SH::H, INFL>(L.segs, 2 * np, L.act, L.outb, OUT_STORE, pre)) return false;
  }
  __syncthreads();
  uint64_t* mll = wsp<uint64_t>(a, a.off.m);
  int base = 0;
  for (int p = 0; p < np; p++) {
    const int n = pc[p].j1 - pc[p].j0;
    for (int j = tid_opaque(); j < n; j += BLOCK)
      ll_put_f32(mll + (size_t)pc[p].slot * SH::INTER + pc[p].j0 + j, silu_f(L.outb[base + j]) * L.outb[base + n + j],
                 st.k1);
    base += 2 * n;
  }
  return true;
}

template <class SH>
__device__ __forceinline__ bool stage_ffn(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  const int w = cx.w, nwg = cx.nwg;
  const uint32_t k1 = st.k1;
  RegVec<SH::H> gam;
  gam.load(Ly.ffn_norm);
  // router workgroups: their router row, loaded ahead of the expert weights
  constexpr int RCH = SH::H / 8, RPT = (RCH + BLOCK - 1) / BLOCK;
  uint4 rrow[SH::MOE ? RPT : 1];
  float rbias = 0.f;   // the expert's selection bias (biased-score router), loaded ahead too
  if constexpr (SH::MOE) {
    if (w < c.E) {
      if (c.router == PLD_ROUTER_SIGMOID_BIAS && tid_opaque() < 4) rbias = gp(Ly.router_bias)[w];
      const uint16_t* rp0 = Ly.router + (size_t)w * SH::H;
#pragma unroll
      for (int k = 0; k < RPT; k++) {
        const int q = tid_opaque() + k * BLOCK;
        rrow[k] = q < RCH ? ld_g16(rp0 + q * 8) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  bool pending = true;
  // read h2, RMSNorm it into LDS; router workgroups publish their logit (fp64)
  auto pre_b = [&]() -> bool {
    if (!pending) return true;
    pending = false;
    if (!ll_fetch<per_for(SH::H)>(cx, reinterpret_cast<uint32_t*>(L.act), wsp<uint64_t>(a, a.off.h2), SH::H, k1, W_H2,
                                  IdxLinear{}, StPad<SH::FP8>{}))
      return false;
    stamp(a, cx, st, TR_H2_READY);
    rmsnorm_reg<SH::H, SH::FP8>(L.act, gam, c.eps, L.red);
    if (w == 0)
      for (int i = tid_opaque(); i < SH::H; i += BLOCK) st_f32(wsp<float>(a, a.off.b_dbg) + i, L.act[apad<SH::FP8>(i)]);
    if constexpr (SH::MOE) {
      if (w < c.E) {
        // logit of expert w (fp64 accumulation) and its selection key: the logit itself
        // (softmax router) or sigmoid(logit) + bias (biased-score router); published as
        // four LL words (logit lo, hi, key lo, hi)
        double s = 0.0;
#pragma unroll
        for (int k = 0; k < RPT; k++) {
          const int q = tid_opaque() + k * BLOCK;
          if (q < RCH) s += dot8_bf16_f64(rrow[k], L.act + apad<SH::FP8>(q * 8));
        }
        s = block_sum(s, L.red);
        if (tid_opaque() < 4) {
          const double key = c.router == PLD_ROUTER_SIGMOID_BIAS
                                 ? (1.0 / (1.0 + exp_f64(-s, L.dk))) + (double)rbias : s;
          const uint64_t bits = (uint64_t)__double_as_longlong(tid_opaque() < 2 ? s : key);
          ll_put(wsp<uint64_t>(a, a.off.logits) + 4 * w + tid_opaque(),
                 (uint32_t)(bits >> (32 * (tid_opaque() & 1))), k1);
        }
        stamp(a, cx, st, TR_RT_LOGIT);
      }
    }
    return true;
  };
  const int j0 = split_at(SH::INTER, nwg, w), j1 = split_at(SH::INTER, nwg, w + 1);
  if constexpr (!SH::MOE) {
    __syncthreads();
    if (tid_opaque() == 0) L.pcs[0] = {0, 0, j0, j1};
    if (!gate_up_list<SH, PLD_IF_SHARED>(a, st, L, j1 > j0 ? 1 : 0, pre_b)) return false;
  } else {
    // shared experts first: they do not depend on the router
    const int np = j1 > j0 ? c.nshared : 0;
    __syncthreads();
    if (tid_opaque() == 0)
      for (int sj = 0; sj < np; sj++) L.pcs[sj] = {c.E + sj, c.topk + sj, j0, j1};
    if (!gate_up_list<SH, PLD_IF_SHARED>(a, st, L, np, pre_b)) return false;
    if (!pre_b()) return false;
    stamp(a, cx, st, TR_SHARED_GEMV);
    // router top-k (every workgroup computes the same selection)
    double* lk = reinterpret_cast<double*>(L.outb);   // [E][2] (logit, key); outb is free here
    if (!ll_fetch<per_for(4 * 512)>(cx, reinterpret_cast<uint32_t*>(lk), wsp<uint64_t>(a, a.off.logits), 4 * c.E, k1,
                                    W_RT))
      return false;
    stamp(a, cx, st, TR_RT_READY);
    // Top-k. The keys become order-preserving 64-bit integers
    // (x >= 0: bits | 2^63, x < 0: ~bits; -0 folded into +0). With many experts one wave
    // selects them in order: lane l holds experts l, l + 64, ... and its best remaining
    // one; each round takes the wave-wide largest (key, lowest index on ties) with DPP
    // moves and the winning lane moves to its next. Both ways place the expert of rank r
    // at position r.
    const bool sig = c.router == PLD_ROUTER_SIGMOID_BIAS;
    if (c.E <= RT_RANK_MAX) {
      // few experts: each expert's rank = #{j : key_j > key_e or (key_j == key_e and
      // j < e)}, its comparisons split over P = BLOCK / E thread partitions; expert e
      // takes position rank(e) when that is < topk
      uint64_t* uk = reinterpret_cast<uint64_t*>(L.outc);         // [E] keys (outc is free here)
      int* rk = reinterpret_cast<int*>(uk + c.E);                  // [P][E] partial ranks
      for (int e = tid_opaque(); e < c.E; e += BLOCK) {
        const double ke = lk[2 * e + 1];
        const uint64_t bb = (uint64_t)__double_as_longlong(ke == 0.0 ? 0.0 : ke);
        uk[e] = (bb >> 63) ? ~bb : (bb | (1ull << 63));
      }
      __syncthreads();
      // E is a power of two dividing BLOCK here; P partitions of E / P comparisons each
      const int P = min(BLOCK / c.E, c.E);
      const int seg = c.E / P;
      const int tid = tid_opaque();
      const int e = tid % c.E, p = tid / c.E;
      if (p < P) {
        const uint64_t ue = uk[e];
        int rank = 0;
        for (int j = p * seg; j < (p + 1) * seg; j++) {
          const uint64_t uj = uk[j];
          rank += (uj > ue || (uj == ue && j < e)) ? 1 : 0;
        }
        rk[p * c.E + e] = rank;
      }
      __syncthreads();
      for (int ee = tid; ee < c.E; ee += BLOCK) {
        int rr = 0;
        for (int pp = 0; pp < P; pp++) rr += rk[pp * c.E + ee];
        if (rr < c.topk) L.isel[rr] = ee;
      }
    } else if (tid_opaque() < 64) {
      // NS slots per lane, a compile-time count (4 up to 256 experts): the unused slots
      // hold key 0, which never wins, so every loop below is branch-free
      auto select = [&](auto ns_tag) {
        constexpr int NS = decltype(ns_tag)::value;
        const int lane = tid_opaque();
        uint64_t ks[NS];   // 0: no expert, or already taken (no score's key is 0)
#pragma unroll
        for (int i = 0; i < NS; i++) {
          const int e = lane + 64 * i;
          const double ke = e < c.E ? lk[2 * e + 1] : 0.0;
          const uint64_t bb = (uint64_t)__double_as_longlong(ke == 0.0 ? 0.0 : ke);
          ks[i] = e < c.E ? ((bb >> 63) ? ~bb : (bb | (1ull << 63))) : 0ull;
        }
        for (int r = 0; r < c.topk; r++) {
          // this lane's best remaining expert (strict > keeps the lower index on ties)
          uint64_t b = ks[0];
          uint32_t bi = 0u;
#pragma unroll
          for (int i = 1; i < NS; i++) {
            const bool gt = ks[i] > b;
            b = gt ? ks[i] : b;
            bi = gt ? (uint32_t)i : bi;
          }
          // wave-wide largest key (DPP moves; a lane keeps its own value where a move
          // does not write it)
          uint64_t m = b;
          auto step = [&](auto ctrl_tag) {
            constexpr int CTRL = decltype(ctrl_tag)::value >> 4, RM = decltype(ctrl_tag)::value & 0xf;
            const uint64_t o = ((uint64_t)dpp_keep_u32<CTRL, RM>((uint32_t)(m >> 32)) << 32) |
                               dpp_keep_u32<CTRL, RM>((uint32_t)m);
            m = o > m ? o : m;
          };
          step(std::integral_constant<int, (0xB1 << 4) | 0xf>{});
          step(std::integral_constant<int, (0x4E << 4) | 0xf>{});
          step(std::integral_constant<int, (0x141 << 4) | 0xf>{});
          step(std::integral_constant<int, (0x140 << 4) | 0xf>{});
          step(std::integral_constant<int, (0x142 << 4) | 0xa>{});
          step(std::integral_constant<int, (0x143 << 4) | 0xc>{});
          const uint64_t K = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(m >> 32), 63) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)m, 63);
          // the expert: the lowest index among the lanes holding that key
          const uint32_t mye = (uint32_t)lane + 64u * bi;
          const bool hold = b == K;
          const uint64_t hm = __ballot(hold);
          uint32_t ee;
          if (__popcll(hm) == 1) ee = (uint32_t)__builtin_amdgcn_readlane((int)mye, __ffsll((unsigned long long)hm) - 1);
          else ee = wave_minmax_u32<false>(hold ? mye : 0xffffffffu);
#pragma unroll
          for (int i = 0; i < NS; i++) ks[i] = (mye == ee && bi == (uint32_t)i) ? 0ull : ks[i];
          if (lane == 0) L.isel[r] = (int)ee;
        }
      };
      if (c.E <= 256) select(std::integral_constant<int, 4>{});
      else select(std::integral_constant<int, RT_SLOTS>{});
    }
    __syncthreads();
    stamp(a, cx, st, TR_TOPK);
    // gates: softmax over the selected logits, or sigmoid scores normalised over the selection
    double* num = reinterpret_cast<double*>(L.outc);
    if (tid_opaque() < c.topk) {
      const double r = lk[2 * L.isel[tid_opaque()]];
      num[tid_opaque()] = sig ? 1.0 / (1.0 + exp_f64(-r, L.dk)) : exp_f64(r - lk[2 * L.isel[0]], L.dk);
    }
    __syncthreads();
    if (tid_opaque() < c.topk) {
      double gsum = 0.0;
      for (int j = 0; j < c.topk; j++) gsum += num[j];
      L.fgate[tid_opaque()] = (float)(num[tid_opaque()] / gsum);
    }
    __syncthreads();
    if (w == 0 && tid_opaque() < c.topk) {
      st_u32(reinterpret_cast<uint32_t*>(wsp<int>(a, a.off.sel)) + tid_opaque(), (uint32_t)L.isel[tid_opaque()]);
      st_f32(wsp<float>(a, a.off.gates) + tid_opaque(), L.fgate[tid_opaque()]);
    }
    // routed experts: this workgroup's share of the topk*inter (slot, row) pairs, one list
    const int tot = c.topk * SH::INTER;
    const int i0 = split_at(tot, nwg, w), i1 = split_at(tot, nwg, w + 1);
    // (every thread counts the pieces; thread 0 writes them; the previous list's readers
    // are past the __syncthreads that follows the gates)
    int nr = 0;
    for (int s = i0 / SH::INTER; s < c.topk && s * SH::INTER < i1 && nr < MAX_PIECES; s++) {
      const int lo = max(i0, s * SH::INTER) - s * SH::INTER, hi = min(i1, (s + 1) * SH::INTER) - s * SH::INTER;
      if (lo < hi) {
        if (tid_opaque() == 0) L.pcs[nr] = {L.isel[s], s, lo, hi};
        nr++;
      }
    }
    if (!gate_up_list<SH, PLD_IF_ROUTED>(a, st, L, nr, NoPre{})) return false;
  }
  stamp(a, cx, st, TR_M_STORED);
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
    if (!ll_fetch<per_for(SH::INTER * MAX_SEGS)>(cx, reinterpret_cast<uint32_t*>(L.act), wsp<uint64_t>(a, a.off.m),
                                                  c.slots * SH::INTER, st.k1, W_M, IdxLinear{}, StPad<SH::FP8>{}))
      return false;
    stamp(a, cx, st, TR_M_READY);
    return true;
  };
  {
    // all slots' rows [r0, r1) as one list; slot s reads activation m_s
    constexpr size_t RB = SH::LUTX ? (size_t)SH::INTER * 3 / 8 : (size_t)SH::INTER * (SH::FP8 ? 1 : 2);
    seg_begin();
    for (int s = 0; s < c.slots; s++) {
      const int expert = !SH::MOE ? 0 : (s < c.topk ? L.isel[s] : c.E + (s - c.topk));
      const size_t bo = (size_t)expert * Ly.dn_slot_bytes + (size_t)r0 * RB;
      const float* sd;
      if constexpr (SH::LUTX)
        sd = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(Ly.w_down.s) + expert * Ly.dn_slot_cb);
      else
        sd = SH::FP8 ? Ly.w_down.s + (size_t)expert * Ly.dn_slot_scales : nullptr;
      seg_set(L, s, Ly.w_down.w + bo, sd, r1 - r0, r0, apad<SH::FP8>(s * SH::INTER), 1.f);
    }
    seg_end();
    if constexpr (SH::LUTX) {
      if (!gemv_list_lut<SH::INTER, PLD_LUT_ITEMS>(L.segs, r1 > r0 ? c.slots : 0, L.act, L.outb, OUT_STORE, pre_m))
        return false;
    } else {
      if (!gemv_list<SH::FP8, SH::INTER, PLD_IF_DOWN>(L.segs, r1 > r0 ? c.slots : 0, L.act, L.outb, OUT_STORE, pre_m))
        return false;
    }
  }
  stamp(a, cx, st, TR_DOWN_GEMV);
  if (!pre_m()) return false;
  stamp(a, cx, st, TR_DOWN_EPI);
  __syncthreads();
  // f_r = sum_s gate_s * down_s[r] (fixed slot order)
  {
    const int nr = r1 - r0;
    for (int r = tid_opaque(); r < nr; r += BLOCK) {
      float f = 0.f;
      for (int s = 0; s < c.slots; s++) f += ((!SH::MOE || s >= c.topk) ? 1.0f : L.fgate[s]) * L.outb[s * nr + r];
      L.outc[r] = f;
      st_f32(wsp<float>(a, a.off.f_dbg) + r0 + r, f);   // debug copy of this workgroup's rows of f
    }
  }
  __syncthreads();
  // out = h2 + f, rounded to bf16: LL words of bf16 pairs (next step's input)
  uint64_t* xll = wsp<uint64_t>(a, a.off.x);
  for (int r = r0 + 2 * tid_opaque(); r < r1; r += 2 * BLOCK) {
    const uint32_t lo = f32_to_bf16(L.h2res[r - r0] + L.outc[r - r0]);
    const uint32_t hi = f32_to_bf16(L.h2res[r + 1 - r0] + L.outc[r + 1 - r0]);
    ll_put(xll + r / 2, lo | (hi << 16), st.k1);
    if (out_hidden) gp(reinterpret_cast<uint32_t*>(out_hidden))[r / 2] = lo | (hi << 16);
  }
  stamp(a, cx, st, TR_DOWN_DONE);
  return true;
}

// ------------------------------------------------------------------ sampling noise
// Gumbel noise g = -log(-log u) of token i at the step of position pos. u comes from a
// counter-based SplitMix64 stream (Steele, Lea and Flood, "Fast splittable pseudorandom
// number generators", OOPSLA 2014; the output mixer of Vigna's splitmix64.c), mod 2^64
// with G = 0x9E3779B97F4A7C15: k = mix(seed * G + pos), r = mix(k + (i + 1) * G),
// u = (2 * (r >> 12) + 1) * 2^-53, exact in fp64 and never 0 or 1. The sampled token is
// argmax_i(logit_i / T + g_i) in fp64 (ties to the lower id), a sample of softmax(logits / T).
__device__ __forceinline__ uint64_t splitmix_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__device__ __noinline__ double gumbel_noise(uint64_t seed, int pos, int i) {
  const uint64_t G = 0x9E3779B97F4A7C15ull;
  const uint64_t k = splitmix_mix(seed * G + (uint64_t)(uint32_t)pos);
  const uint64_t r = splitmix_mix(k + (uint64_t)(uint32_t)(i + 1) * G);
  const double u = ((double)(r >> 12) * 2.0 + 1.0) * 0x1p-53;
  return -log(-log(u));
}

// ------------------------------------------------------------------ LM head + greedy argmax / sampling
// logits = W_head RMSNorm(x; gamma_final) for this workgroup's vocab rows, accumulated in
// fp64: an FP8 code times its fp32 block scale times an fp64 activation is exact in fp64,
// so the logits equal an fp64 evaluation up to summation rounding and the argmax is
// decided in fp64. The global argmax (lowest token id on ties) is formed from every
// workgroup's local best, published as LL words; every workgroup derives the same token,
// whose embedding row is the next token's input.
template <class SH>
__device__ __forceinline__ bool stage_head(Ctx& cx, const KArgs& a, const Step& st, Lds& L, int t, int* token) {
  const KCfg& c = a.c;
  constexpr int H = SH::H;
  constexpr int EPC = 16, CHUNKS = H / EPC, CPL = CHUNKS / 64, SBK = (H + 127) / 128;
  static_assert(SH::FP8 && CHUNKS % 64 == 0, "FP8 head with whole 64-lane rows");
  const int V = c.vocab, nwg = cx.nwg, w = cx.w;
  const uint32_t k1 = st.k1;
  const int r0 = split_at(V, nwg, w), r1 = split_at(V, nwg, w + 1), nr = r1 - r0;
  const int tid = tid_opaque(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  RegVec<H> gf;
  gf.load(a.fnorm);
  constexpr int U = 2;                                   // rows in flight per wave
  const int nrw = max(0, (nr - wave + NWAVES - 1) / NWAVES);   // rows r0 + wave + i*NWAVES
  uint4 buf[U][CPL];
  float sc[U][CPL];
  auto issue = [&](int u, int i) {   // unconditional: rows past the wave's last are clamped
    const int r = r0 + wave + min(i, max(nrw - 1, 0)) * NWAVES;
    const uint8_t* p = a.head.w + (size_t)min(r, V - 1) * H + lane * 16;
    const PLD_GLOBAL float* srow = gp(a.head.s) + (size_t)(min(r, V - 1) >> 7) * SBK;
#pragma unroll
    for (int j = 0; j < CPL; j++) {
      buf[u][j] = ld_stream16(p + (size_t)j * 64 * 16);
      sc[u][j] = srow[((j * 64 + lane) * 16) >> 7];
    }
  };
#pragma unroll
  for (int u = 0; u < U; u++) issue(u, u);
  // input: x of the token's last layer (LL), RMSNorm in fp64. Stored swizzled: element
  // (chunk c = 64 j + l, offset e) at ((j * 16 + e) * 64 + l), so that the 64 lanes of a
  // wave (chunk l of chunk group j) read 64 consecutive doubles (no LDS bank conflicts).
  double* dact = reinterpret_cast<double*>(L.act);   // [H]
  auto swz = [](int i) { const int c = i >> 4; return ((c >> 6) * 16 + (i & 15)) * 64 + (c & 63); };
  if (!ll_fetch<per_for(H / 2)>(cx, L.stage, wsp<uint64_t>(a, a.off.x), H / 2, k1, W_X)) return false;
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < (H / 2 + BLOCK - 1) / BLOCK; k++) {
    const int i = tid + k * BLOCK;
    if ((H / 2) % BLOCK == 0 || i < H / 2) {
      const uint32_t v = L.stage[i];
      const double x0 = bf_lo(v), x1 = bf_hi(v);
      ss += x0 * x0 + x1 * x1;
    }
  }
  ss = block_sum(ss, L.red);
  const double rr = 1.0 / sqrt(ss / (double)H + c.eps);
#pragma unroll
  for (int k = 0; k < RegVec<H>::K; k++) {
    const int i = tid + k * BLOCK;
    if (H % BLOCK == 0 || i < H) {
      const uint32_t v = L.stage[i >> 1];
      const double x = (i & 1) ? bf_hi(v) : bf_lo(v);
      dact[swz(i)] = (x * rr) * (double)gf.v[k];
    }
  }
  __syncthreads();
  stamp(a, cx, st, TR_HEAD_READY);
  double* lg = reinterpret_cast<double*>(L.outb);    // [nr]
  for (int i0 = 0; i0 < nrw; i0 += U) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int i = i0 + u;
      double acc = 0.0;
#pragma unroll
      for (int j = 0; j < CPL; j++) {
        const double* av = dact + j * 16 * 64 + lane;   // element e of this lane's chunk at av[e * 64]
        const uint32_t d[4] = {buf[u][j].x, buf[u][j].y, buf[u][j].z, buf[u][j].w};
        const double s = (double)sc[u][j];
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)d[q], false);
          const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)d[q], true);
          acc = fma((double)lo.x * s, av[(4 * q + 0) * 64], acc);
          acc = fma((double)lo.y * s, av[(4 * q + 1) * 64], acc);
          acc = fma((double)hi.x * s, av[(4 * q + 2) * 64], acc);
          acc = fma((double)hi.y * s, av[(4 * q + 3) * 64], acc);
        }
      }
      issue(u, i + U);
      acc = dpp_sum64_f64(acc);
      if (lane == 63 && i < nrw) lg[wave + i * NWAVES] = acc;
    }
  }
  __syncthreads();
  stamp(a, cx, st, TR_HEAD_GEMV);
  if (a.out_logits)
    for (int i = tid; i < nr; i += BLOCK) gp(a.out_logits)[(size_t)t * V + r0 + i] = (float)lg[i];
  // best of this workgroup: (key desc, token id asc); key = logit (greedy) or logit / T + g
  auto better = [](double v, int i, double bv, int bi) { return v > bv || (v == bv && i < bi); };
  uint64_t* am = wsp<uint64_t>(a, a.off.amax);
  if (wave == 0) {
    double bv = -INFINITY;
    int bi = 0x7fffffff;
    const double temp = a.temperature;
    for (int i = lane; i < nr; i += 64) {
      const double key = temp > 0.0 ? lg[i] / temp + gumbel_noise(a.sample_seed, st.pos, r0 + i) : lg[i];
      if (better(key, r0 + i, bv, bi)) { bv = key; bi = r0 + i; }
    }
    for (int off = 32; off >= 1; off >>= 1) {
      const double ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) {
      const uint64_t b = (uint64_t)__double_as_longlong(bv);
      ll_put(am + 3 * w, (uint32_t)b, k1);
      ll_put(am + 3 * w + 1, (uint32_t)(b >> 32), k1);
      ll_put(am + 3 * w + 2, (uint32_t)bi, k1);
    }
  }
  // the global best from every workgroup's candidate (the same token in every workgroup)
  uint32_t* cand = L.stage;   // [3 * nwg]
  if (!ll_fetch<per_for(3 * 512)>(cx, cand, am, 3 * nwg, k1, W_AMAX)) return false;
  if (wave == 0) {
    double bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int g = lane; g < nwg; g += 64) {
      const double v = __longlong_as_double((long long)(((uint64_t)cand[3 * g + 1] << 32) | cand[3 * g]));
      const int i = (int)cand[3 * g + 2];
      if (better(v, i, bv, bi)) { bv = v; bi = i; }
    }
    for (int off = 32; off >= 1; off >>= 1) {
      const double ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) L.isel[0] = bi;
  }
  __syncthreads();
  *token = L.isel[0];
  __syncthreads();
  if (w == 0 && tid == 0 && a.out_tokens) gp(a.out_tokens)[t] = *token;
  stamp(a, cx, st, TR_TOKEN);
  return true;
}

template <class SH>
__global__ void __launch_bounds__(BLOCK, 1) k_decode_gqa(KArgs a) {
  extern __shared__ float lds_raw[];
  Ctx cx;
  cx.budget = a.budget;
  cx.w = blockIdx.x;
  cx.nwg = gridDim.x;
  cx.status = wsp<uint32_t>(a, a.off.status);
  cx.wacc = nullptr;
  const DLayer* layers = wsp<DLayer>(a, a.off.layers);
  if ((a.hooks & PLD_HOOK_DROP_WG0) && cx.w == 0) return;   // test hook: a producer that never publishes
  {
    Lds L0 = carve(lds_raw, a.c);
    if (tid_opaque() < TR_SLOTS) L0.tr[tid_opaque()] = 0;
    exp_f64_init(L0.dk);
    __syncthreads();
  }
  int token = a.in_token;   // greedy decode loop: the token whose embedding feeds the next layer 0
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
      st.emb_row = (li == 0 && a.head_on && token >= 0) ? a.embed + (size_t)token * SH::H : nullptr;
      const bool last = (t == a.n_tokens - 1) && (li == a.n_layers - 1);
      // The workspace base is made opaque for every step: per-lane addresses derived from
      // it are then recomputed inside the step instead of being hoisted out of the loop
      // and held (spilled) across all stages.
      KArgs as = a;
      asm volatile("" : "+s"(as.ws));
      // the same for the LDS carve (a 32-bit offset, so the pointers stay LDS pointers)
      uint32_t lds0 = 0;
      asm volatile("" : "+s"(lds0));
      Lds L = carve(lds_raw + lds0, a.c);
      st.tr = L.tr;
      cx.wacc = (a.trace && st.idx < a.trace_steps) ? L.tr + TR_WAIT : nullptr;
      stamp(as, cx, st, TR_START);
      PLD_TEST_DELAY(a, cx.w, st.idx, 0);
      if (!stage_qkv_gqa<SH>(cx, as, st, L)) return;
      PLD_TEST_DELAY(a, cx.w, st.idx, 1);
      if (!attention_gqa<SH>(cx, as, st, L)) return;
      if (!stage_wo<SH>(cx, as, st, L)) return;
      PLD_TEST_DELAY(a, cx.w, st.idx, 2);
      if (!stage_ffn<SH>(cx, as, st, L)) return;
      PLD_TEST_DELAY(a, cx.w, st.idx, 3);
      if (!stage_down<SH>(cx, as, st, L, last ? as.out_hidden : nullptr)) return;
      if constexpr (SH::FP8) {
        if (a.head_on && li == a.n_layers - 1 && !stage_head<SH>(cx, as, st, L, t, &token)) return;
      }
      trace_flush(as, cx, st);
    }
  }
}

#include "pld_mla.hpp"
#include "pld_kda.hpp"
#include "pld_batch.hpp"

typedef void (*KernelFn)(KArgs);

// The compiled shapes: the tiny dense MHA layer (hidden 256, 4x64 heads, FFN 1024) and
// the GQA MoE layer (hidden 4096, 32 q / 8 kv heads x 128, 64 experts of width 1536).
using ShapeTinyDense = GqaShape<256, 4, 4, 64, 1024, false, false, 1, 2>;
using ShapeGqaMoe = GqaShape<4096, 32, 8, 128, 1536, false, true, 9, 33>;
// the FP8 MLA MoE layer: hidden 6144, 64 heads, q_lora 1536, kv_lora 512 + rope 64,
// nope 128, v 128, 256 experts of width 2048 (biased-score router)
using ShapeMlaFp8 = MlaShape<6144, 64, 1536, 512, 64, 128, 128, 2048, true, true, false, 0, 0, 16>;
// the sparse MLA MoE layer: hidden 4096, 32 heads, the same latent sizes, bf16 weights,
// indexer of 8 heads x 64 dims, 64 experts of width 1536 (softmax router)
using ShapeSparseMla = MlaShape<4096, 32, 1536, 512, 64, 128, 128, 1536, false, true, true, 8, 64>;
// the KDA MoE layer: hidden 6144, 32 KDA heads x 128, decay rank 128, convolution width 4,
// FP8 weights, 256 experts of width 2048 (biased-score router)
using ShapeKda = KdaShape<6144, 32, 128, 128, 4, 2048, true, true>;
// the FP8 MLA MoE layer with LUT3 expert matrices (3-bit indices into 8-entry E4M3 codebooks)
using ShapeMlaLut = MlaShape<6144, 64, 1536, 512, 64, 128, 128, 2048, true, true, false, 0, 0, 16, true>;

template <class SH>
static bool matches_kda(const pld_config* c) {
  return c->attn_kind == PLD_ATTN_KDA && c->hidden == SH::H && c->n_heads == SH::NH && c->head_dim == SH::D &&
         c->kda_rank == SH::R && c->conv_width == SH::CW && c->inter == SH::INTER &&
         (c->wfmt == PLD_WFMT_FP8_BLOCK128) == SH::FP8 && (c->ffn_kind == PLD_FFN_MOE) == SH::MOE;
}

template <class SH>
static bool matches(const pld_config* c) {
  return c->attn_kind == PLD_ATTN_GQA && c->hidden == SH::H && c->n_heads == SH::NH && c->n_kv_heads == SH::NKV &&
         c->head_dim == SH::HD && c->inter == SH::INTER && (c->wfmt == PLD_WFMT_FP8_BLOCK128) == SH::FP8 &&
         (c->ffn_kind == PLD_FFN_MOE) == SH::MOE;
}

template <class SH>
static bool matches_mla(const pld_config* c) {
  return c->attn_kind == PLD_ATTN_MLA && c->hidden == SH::H && c->n_heads == SH::NH && c->q_lora == SH::QL &&
         c->kv_lora == SH::KL && c->rope_dim == SH::RD && c->nope_dim == SH::ND && c->v_dim == SH::VD &&
         c->inter == SH::INTER && (c->wfmt == PLD_WFMT_FP8_BLOCK128) == SH::FP8 &&
         (c->ffn_kind == PLD_FFN_MOE) == SH::MOE && (c->index_topk > 0) == SH::SPARSE &&
         (!SH::SPARSE || (c->index_heads == SH::IH && c->index_dim == SH::ID)) &&
         (c->expert_wfmt == PLD_WFMT_LUT3) == SH::LUTX;
}

// heads per MLA attention workgroup of the compiled shape the configuration selects
static int mla_hpw(const pld_config* c) {
  if (matches_mla<ShapeMlaFp8>(c)) return ShapeMlaFp8::HPW;
  if (matches_mla<ShapeMlaLut>(c)) return ShapeMlaLut::HPW;
  if (matches_mla<ShapeSparseMla>(c)) return ShapeSparseMla::HPW;
  return 0;
}

static KernelFn pick_kernel(const pld_config* c) {
  if (matches<ShapeTinyDense>(c)) return k_decode_gqa<ShapeTinyDense>;
  if (matches<ShapeGqaMoe>(c)) return k_decode_gqa<ShapeGqaMoe>;
  if (matches_mla<ShapeMlaFp8>(c)) return k_decode_mla<ShapeMlaFp8>;
  if (matches_mla<ShapeSparseMla>(c)) return k_decode_mla<ShapeSparseMla>;
  if (matches_mla<ShapeMlaLut>(c)) return k_decode_mla<ShapeMlaLut>;
  if (matches_kda<ShapeKda>(c)) return k_decode_kda<ShapeKda>;
  return nullptr;
}

// the batched kernel of a configuration (the FP8 MLA MoE shape with a head) for a verify
// (batch = false) or a batch decode, or null
static KernelFn pick_verify(const pld_config* c, bool batch = false) {
  if (matches_mla<ShapeMlaFp8>(c) && c->vocab > 0) return batch ? k_verify_mla<ShapeMlaFp8, 1> : k_verify_mla<ShapeMlaFp8, 0>;
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
  KernelFn vfn;            // batched verify kernel (cfg.max_query >= 2), else null
  KernelFn bfn;            // batch decode kernel (with vfn), else null
  size_t vlds_bytes;
  int device;
  uint64_t* trace;
  int trace_steps;
  const uint16_t* embed;   // LM head (vocab > 0)
  const float* fnorm;
  DMat head;
  int hooks;               // test hooks for the next launches (PLD_HOOK_DROP_WG0 lasts one launch)
  uint32_t hook_seed;
  bool is_static;          // made by decode_layer_init_static: library storage, never freed
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
  k->krank = c->kda_rank; k->cwidth = c->conv_width;
  if (c->hidden <= 0 || c->n_heads <= 0 || c->max_seq <= 0 || c->inter <= 0 || !(c->eps >= 0.0)) return PLD_E_INVALID;
  // every size field within bounds that keep the sizing arithmetic below in range (unused
  // fields of another layer kind included), a finite eps and RoPE base
  {
    const int32_t dims[] = {c->hidden, c->n_heads, c->n_kv_heads, c->head_dim, c->q_lora, c->kv_lora, c->rope_dim,
                            c->nope_dim, c->v_dim, c->index_heads, c->index_dim, c->index_topk, c->inter,
                            c->n_experts, c->top_k, c->n_shared, c->kda_rank, c->conv_width};
    for (int32_t d : dims)
      if (d < 0 || d > (1 << 16)) return PLD_E_INVALID;
    if (c->n_heads > 1024 || c->n_kv_heads > 1024 || c->head_dim > 1024 || c->max_seq > (1 << 22) ||
        c->vocab > (1 << 22) || nwg < 1 || nwg > 4096 || !(c->eps <= 1.0) || !(c->rope_base > 0.0) ||
        !(c->rope_base < 1e300))
      return PLD_E_INVALID;
  }
  if (c->wfmt != PLD_WFMT_BF16 && c->wfmt != PLD_WFMT_FP8_BLOCK128) return PLD_E_UNSUPPORTED;
  if (c->expert_wfmt != 0 && c->expert_wfmt != PLD_WFMT_LUT3) return PLD_E_UNSUPPORTED;
  // LUT3 experts: whole 16-lane rows of 128-weight groups for both reduction lengths
  if (c->expert_wfmt == PLD_WFMT_LUT3 && (c->ffn_kind != PLD_FFN_MOE || c->wfmt != PLD_WFMT_FP8_BLOCK128 ||
                                          c->hidden % 2048 || c->inter % 2048 || c->inter % 8 || c->hidden % 8))
    return PLD_E_UNSUPPORTED;
  if (nwg < NXCD || nwg % NXCD) return PLD_E_UNSUPPORTED;
  if (c->ffn_kind == PLD_FFN_DENSE) {
    k->slots = 1;
  } else if (c->ffn_kind == PLD_FFN_MOE) {
    if (c->n_experts < 8 || c->n_experts > nwg || c->n_experts > 64 * RT_SLOTS || c->n_experts % 8 ||
        (c->n_experts <= RT_RANK_MAX && BLOCK % c->n_experts))
      return PLD_E_UNSUPPORTED;
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
    // One LL buffer per activation is safe when every workgroup that reads a buffer is
    // an ancestor of its next writer: every workgroup must publish some q/k/v rows and
    // some expert activations (m) each step.
    if ((c->n_heads + 2 * c->n_kv_heads) * c->head_dim / 2 < nwg) return PLD_E_UNSUPPORTED;
    if (c->inter < nwg) return PLD_E_UNSUPPORTED;
    k->cpg = nwg / c->n_kv_heads;
    k->chmax = (c->max_seq + k->cpg - 1) / k->cpg + 1;
    const int R = (c->n_heads + 2 * c->n_kv_heads) * c->head_dim;
    // attention: q [G*HD] + new k/v row [HD] + scores [G*chmax] + wave sums [8*G*HD] + (m, l);
    // merge staging: at most G*HD/cpg + 1 dims of cpg chunks, (m, l) and weights of two heads
    // (the GEMV inputs in their LDS layout: padded for FP8 weights)
    const bool pad = c->wfmt == PLD_WFMT_FP8_BLOCK128;
    auto ap = [pad](int n) { return pad ? apad<true>(n) : n; };
    using ll = long long;
    const ll act = std::max<ll>({ap(c->hidden), ap(c->n_heads * c->head_dim), ap(k->slots * c->inter),
                                 2LL * k->G * c->head_dim + c->head_dim + (ll)k->G * k->chmax +
                                     (ll)NWAVES * k->G * c->head_dim + 2 * k->G + 8,
                                 (ll)k->cpg * (k->G * c->head_dim / k->cpg + 1) + 8LL * k->cpg + 8});
    if (act > (1 << 20)) return PLD_E_UNSUPPORTED;
    k->act_floats = (int)al((size_t)act, 64);
    k->stage_words = (int)al(c->hidden / 2 + 2, 64);
    int outb = std::max({R / nwg + 4, k->slots * (c->hidden / nwg + 4), 2 * ((k->slots * c->inter) / nwg + 2),
                         2 * (c->inter / nwg + 2) * std::max(1, c->n_shared), 4 * c->n_experts + 4,
                         2 * c->n_experts + BLOCK});
    k->outb_floats = (int)al(outb, 64);
    if (lds_bytes_for(k->act_floats, k->stage_words, k->outb_floats) > 160 * 1024) return PLD_E_UNSUPPORTED;
    k->rdim = c->head_dim;
  } else if (c->attn_kind == PLD_ATTN_MLA) {
    if (!pick_kernel(c)) return PLD_E_UNSUPPORTED;
    const int HPW = mla_hpw(c), NH = c->n_heads, KL = c->kv_lora, LAT = c->kv_lora + c->rope_dim, VD = c->v_dim;
    const int nhg = NH / HPW;
    if (NH % HPW || nwg % nhg) return PLD_E_UNSUPPORTED;
    k->cpg = nwg / nhg;                            // attention chunks per head group
    k->rdim = c->rope_dim;
    // absorb / merge: cpw outputs of one head per workgroup, whole 16-byte chunks, <= 4 row passes
    if ((NH * KL) % nwg) return PLD_E_UNSUPPORTED;
    k->cpw = NH * KL / nwg;
    const int epc = c->wfmt == PLD_WFMT_FP8_BLOCK128 ? 16 : 8;
    if (KL % k->cpw || k->cpw % epc || BLOCK % k->cpw || c->nope_dim > 4 * (BLOCK / (k->cpw / epc)))
      return PLD_E_UNSUPPORTED;
    // W_UV: each workgroup's rows inside one head
    if ((NH * VD) % nwg || VD % (NH * VD / nwg)) return PLD_E_UNSUPPORTED;
    // one LL buffer per activation: every workgroup publishes rows in every stage
    if (c->q_lora + LAT < nwg || c->inter < nwg || c->hidden / 2 < nwg) return PLD_E_UNSUPPORTED;
    const bool sparse = c->index_topk > 0;
    const int TB = 32, CSTR = LAT + 4;
    // sparse: the chunk's selected-row list follows the attention scratch
    const int srows_max = sparse ? (std::min(c->index_topk, c->max_seq) + k->cpg - 1) / k->cpg : 0;
    const int attn_bytes = 2 * 16 * CSTR + 2 * 2 * TB * CSTR + 2 * 16 * TB + 4 * (8 * 256 + 16) + 2 * LAT + 4 * LAT +
                           4 * srows_max;
    // (the GEMV inputs in their LDS layout: padded for FP8 weights)
    const bool pad = c->wfmt == PLD_WFMT_FP8_BLOCK128;
    auto ap = [pad](int n) { return pad ? apad<true>(n) : n; };
    int act = std::max({ap(c->hidden), ap(c->q_lora), ap(k->slots * c->inter), ap(NH * VD), ap(KL),
                        (attn_bytes + 3) / 4 + 16,
                        c->nope_dim + (BLOCK / (k->cpw / epc) + 1) * k->cpw + BLOCK,   // absorb: q_nope, partials, sums
                        k->cpg * k->cpw + 3 * k->cpg + 8 + BLOCK});
    if (sparse) {
      // indexer: 8 heads x 64 dims (4 lanes x 2 heads per token); selection: every scoring
      // workgroup's list in LDS, keys per thread on the all-token path; selected rows per
      // chunk (LL fetch, one pass)
      if (c->index_heads != 8 || c->index_dim != 64 || c->index_topk < 1 || c->index_topk > SEL_STAGE_MAX)
        return PLD_E_UNSUPPORTED;
      if (c->max_seq > SEL_MAXJ * BLOCK || c->max_seq > SEL_LKMAX * nwg || nwg > SEL_MAXWG || srows_max > BLOCK ||
          srows_max > 8 * TB)
        return PLD_E_UNSUPPORTED;
      const int idx_words = 2 * (c->index_heads * c->index_dim + c->index_heads) + 2 * SEL_LKMAX + SEL_LIST +
                            c->index_heads * c->index_dim / 2 + c->index_heads + c->index_dim + c->index_dim / 4 + 3;
      act = std::max({act, ap(c->q_lora) + 2 * c->q_lora, SEL_LDS_WORDS, idx_words});
      if (c->q_lora + LAT + c->index_heads + c->index_dim < nwg) return PLD_E_UNSUPPORTED;
    }
    k->act_floats = (int)al(act, 64);
    k->stage_words = (int)al(c->hidden / 2 + 2, 64);
    const int rx = c->q_lora + LAT + (sparse ? c->index_heads + c->index_dim : 0);
    const int rq = NH * (c->nope_dim + c->rope_dim) + (sparse ? c->index_heads * c->index_dim : 0);
    const int f64x = sparse ? 2 : 1;   // fp64 row results take two floats
    int outb = std::max({f64x * (rx / nwg + 4), f64x * (rq / nwg + 4), NH * VD / nwg + 4, c->hidden / nwg + 4,
                         k->slots * (c->hidden / nwg + 4), 2 * ((k->slots * c->inter) / nwg + 2),
                         2 * (c->inter / nwg + 2) * std::max(1, c->n_shared), 4 * c->n_experts + 4,
                         2 * c->n_experts + BLOCK});
    k->outb_floats = (int)al(outb, 64);
    if (lds_bytes_for(k->act_floats, k->stage_words, k->outb_floats) > 160 * 1024) return PLD_E_UNSUPPORTED;
  } else if (c->attn_kind == PLD_ATTN_KDA) {
    if (!pick_kernel(c)) return PLD_E_UNSUPPORTED;
    const int NH = c->n_heads, D = c->head_dim, QD = NH * D, R = c->kda_rank;
    const int rows = 4 * QD + R + NH;
    // the state stage: each workgroup owns 16 value columns of one head
    if (nwg != NH * (D / 16)) return PLD_E_UNSUPPORTED;
    // the projection stage: one row per thread, and every workgroup publishes some rows
    if ((rows + nwg - 1) / nwg > BLOCK || rows < nwg || c->inter < nwg || c->hidden / 2 < nwg) return PLD_E_UNSUPPORTED;
    const bool pad = c->wfmt == PLD_WFMT_FP8_BLOCK128;
    auto ap = [pad](int n) { return pad ? apad<true>(n) : n; };
    int act = std::max({ap(c->hidden), ap(QD) + 2 * QD, ap(k->slots * c->inter),
                        2 * D + 16 + R + 4 + NWAVES * 16 + 16 + 4 + 2 * NWAVES + 8});
    k->act_floats = (int)al(act, 64);
    k->stage_words = (int)al(c->hidden / 2 + 2, 64);
    int outb = std::max({rows / nwg + 4, c->hidden / nwg + 4, k->slots * (c->hidden / nwg + 4),
                         2 * ((k->slots * c->inter) / nwg + 2), 2 * (c->inter / nwg + 2) * std::max(1, c->n_shared),
                         4 * c->n_experts + 4, 2 * c->n_experts + BLOCK});
    k->outb_floats = (int)al(outb, 64);
    if (lds_bytes_for(k->act_floats, k->stage_words, k->outb_floats) > 160 * 1024) return PLD_E_UNSUPPORTED;
    k->rdim = 2;   // no RoPE
  } else {
    return PLD_E_UNSUPPORTED;
  }
  if (c->vocab < 0) return PLD_E_INVALID;
  if (c->vocab > 0) {
    // LM head: FP8 block-scaled [vocab, hidden] on the FP8 shapes; every workgroup owns rows
    if (c->wfmt != PLD_WFMT_FP8_BLOCK128 || c->vocab < nwg || (c->hidden / 16) % 64) return PLD_E_UNSUPPORTED;
    if (k->outb_floats < 2 * ((c->vocab + nwg - 1) / nwg) || k->act_floats < 2 * c->hidden ||
        k->stage_words < 3 * nwg)
      return PLD_E_UNSUPPORTED;
  }
  if (c->max_query < 0 || c->max_query > VB || c->max_batch < 0 || c->max_batch > VB) return PLD_E_INVALID;
  if (c->max_query >= 2 || c->max_batch >= 2) {
    // batched verify: the per-workgroup row counts must fit its LDS result areas
    if (!pick_verify(c) || c->n_shared > 4 || c->top_k > 8 || c->n_experts > 256 || k->cpw != 128)
      return PLD_E_UNSUPPORTED;
    auto per = [nwg](long long n) { return (n + nwg - 1) / nwg; };
    // X rows: W_DQ over the first nwq workgroups, W_DKV over the rest (as the batched X stage splits them)
    const long long R = c->q_lora + c->kv_lora + c->rope_dim;
    const long long nwq = std::max(1LL, std::min((long long)nwg - 1, ((long long)nwg * c->q_lora + R / 2) / R));
    const long long hr = 2 * per(c->hidden / 2),
                    xr = nwg < 2 ? R : std::max((c->q_lora + nwq - 1) / nwq, (R - c->q_lora + (nwg - nwq) - 1) / (nwg - nwq));
    const long long qr = 2 * per((long long)c->n_heads * (c->nope_dim + c->rope_dim) / 2);
    const long long ur = per((long long)c->n_heads * c->v_dim), sr = 2 * per(c->inter / 2);
    const int rows = std::max(c->max_query, c->max_batch);
    const long long gr = 2 * (2 * per((long long)rows * c->top_k * c->inter / 2));
    if (hr > 32 || xr > 64 || qr > 64 || ur > 64 || 2 * c->n_shared * sr > 64 ||
        98432 + (long long)VB * gr * 4 > VACT_BYTES || ((long long)c->n_heads * c->v_dim) % nwg)
      return PLD_E_UNSUPPORTED;
    k->vq = rows;
    k->vb = c->max_batch >= 2 ? c->max_batch : 0;
  }
  return PLD_OK;
}

WsOff layout(const KCfg& k, int n_layers) {
  WsOff o;
  size_t p = 0;
  const size_t W = 8;   // LL word
  o.status = p; p += al(64);
  o.x = p; p += al((size_t)(k.H / 2) * W);
  o.q = p; p += al((size_t)std::max(k.nh * k.hd, 1) * W);
  o.kv = p; p += al((size_t)std::max(k.nkv * k.hd, 1) * W);   // k half then v half, bf16 pairs
  o.part = p; p += al((size_t)k.nh * k.cpg * (k.hd + 2) * W);
  o.o = p; p += al((size_t)std::max(k.nh * k.hd, 1) * W);
  o.h2 = p; p += al((size_t)k.H * W);
  o.logits = p; p += al((size_t)std::max(k.E, 1) * 4 * W);
  o.m = p; p += al((size_t)k.slots * k.inter * W);
  if (k.attn == PLD_ATTN_MLA) {
    const size_t LAT = (size_t)k.kv_lora + k.rope;
    o.q = p; p += al((size_t)k.nh * k.nope * W);                     // q_nope
    o.qr = p; p += al((size_t)k.nh * k.rope * W);                    // q_rope (rotated)
    o.cqr = p; p += al((size_t)2 * k.q_lora * W);                    // c_q before its RMSNorm (fp64: 2 words)
    o.ckvr = p; p += al(LAT * W);                                    // c_kv and k_rope before norm / RoPE
    o.qlat = p; p += al((size_t)k.nh * k.kv_lora * W);
    o.part = p; p += al((size_t)k.nh * k.cpg * (k.kv_lora + 2) * W);
    o.olat = p; p += al((size_t)k.nh * k.kv_lora * W);
    o.o = p; p += al((size_t)k.nh * k.vdim * W);
  } else {
    o.cqr = o.ckvr = o.qr = o.qlat = o.olat = 0;
  }
  o.amax = p; p += al((size_t)3 * std::max(k.nwg, 1) * W);   // per-workgroup (logit lo, hi, index)
  if (k.attn == PLD_ATTN_KDA) {
    const int QD = k.nh * k.hd;
    o.kx = p; p += al((size_t)(4 * QD + k.krank + k.nh) * W);   // conv outputs, gate, a_down, beta
  } else {
    o.kx = 0;
  }
  if (k.itopk > 0) {
    o.ixr = p; p += al((size_t)(k.ih + k.idim) * W);       // indexer head weights w and new key k_I (fp32)
    o.qi = p; p += al((size_t)(k.ih * k.idim / 2) * W);    // indexer queries (bf16 pairs)
    o.ilist = p; p += al((size_t)k.nwg * SEL_LIST * W);    // per-workgroup top key high halves, rank order
    o.isel = p; p += al((size_t)k.itopk * W);              // selected rows, ascending
  } else {
    o.ixr = o.qi = o.ilist = o.isel = 0;
  }
  if (k.vq >= 2) {
    const size_t VBW = 8;   // positions per batched step (the kernel's per-position strides)
    const size_t LAT = (size_t)k.kv_lora + k.rope;
    o.vx = p; p += al(VBW * (k.H / 2) * W);
    o.vcqr = p; p += al(VBW * k.q_lora * W);
    o.vckv = p; p += al(VBW * LAT * W);
    o.vqn = p; p += al(VBW * k.nh * k.nope * W);
    o.vqr = p; p += al(VBW * (k.nh * k.rope / 2) * W);
    o.vqlat = p; p += al(VBW * (k.nh * k.kv_lora / 2) * W);
    o.vpart = p; p += al(VBW * k.nh * k.cpg * (k.kv_lora / 2 + VP_ACC) * W);   // [m, l, spare | acc] rows of whole lines
    o.volat = p; p += al(VBW * k.nh * k.kv_lora * W);
    o.vo = p; p += al(VBW * (k.nh * k.vdim / 2) * W);
    o.vh2 = p; p += al(VBW * k.H * W);
    // partial sums over each W_O workgroup's rows (fp64 as two words): sum of h2^2 per
    // position [nwg][VBW], then the router's gamma-weighted dot products [E][nwg][VBW]
    o.vss = p; p += al((size_t)k.nwg * VBW * 2 * W);
    o.vrp = p; p += al((size_t)k.E * k.nwg * VBW * 2 * W);
    o.vhn = p; p += al(VBW * (k.H / 2) * W);   // the normalised FFN operand rows (bf16 pairs)
    o.vlog = p; p += al(VBW * 4 * k.E * W);
    o.vm = p; p += al((size_t)(k.vq * k.topk + k.nshared) * VBW * (k.inter / 2) * W);
    o.vfp = p; p += al((size_t)(k.vq * k.topk + k.nshared) * VBW * k.H * W);   // gated down partials
    o.vamax = p; p += al(VBW * 3 * k.nwg * W);
  } else {
    o.vx = o.vcqr = o.vckv = o.vqn = o.vqr = o.vqlat = o.vpart = o.volat = o.vo = o.vh2 = o.vss = o.vrp = o.vhn =
        o.vlog = o.vm = o.vfp = o.vamax = 0;
  }
  o.ll_end = p;
  if (k.vq >= 2) {
    o.vsel = p; p += al(8 * 8 * 4 * 2);   // per-position top-k experts, then their gates
    o.vf = p; p += al((size_t)8 * k.H * 4);   // per-position FFN output before the residual
  } else {
    o.vsel = o.vf = 0;
  }
  o.sel = p; p += al(64 * 4);
  o.gates = p; p += al(64 * 4);
  o.spec = p; p += al(64 * 4);   // decode_speculative: drafts [16], verify tokens [16], accepted, spare
  o.a_dbg = p; p += al((size_t)k.H * 4);
  o.b_dbg = p; p += al((size_t)k.H * 4);
  o.f_dbg = p; p += al((size_t)k.H * 4);
  if (k.itopk > 0) {
    o.ikh = p; p += al((size_t)k.max_seq * 4);   // indexer score keys, high and low halves
    o.ikl = p; p += al((size_t)k.max_seq * 4);
    o.ilo = p; p += al((size_t)k.nwg * SEL_LIST * 4);   // list entries: low halves and tokens
    o.itok = p; p += al((size_t)k.nwg * SEL_LIST * 4);
  } else {
    o.ikh = o.ikl = o.ilo = o.itok = 0;
  }
  o.rope = p; p += al((size_t)k.max_seq * std::max(k.rdim, 2) * 4);
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
  const int nwg = device_cus(nullptr);
  if (nwg <= 0) return 0;
  return pld_workspace_bytes_for_cus(cfg, n_layers, nwg);
}

size_t pld_workspace_bytes_for_cus(const pld_config* cfg, int32_t n_layers, int32_t n_cus) {
  if (!cfg || n_layers < 1 || n_cus < 1) return 0;
  KCfg k;
  if (derive(cfg, n_cus, &k) != PLD_OK) return 0;
  return layout(k, n_layers).total;
}

}  // extern "C"

namespace {

// RoPE table (cos, sin) of pos * base^(-2i/d) for the interleaved pairs, fp64 -> fp32, written
// to the device in chunks from a fixed host buffer (init allocates nothing).
bool upload_rope(uint8_t* dst, int max_seq, int d, double base) {
  constexpr int CH = 4096;   // floats per chunk
  float buf[CH];
  const size_t total = (size_t)max_seq * d;
  for (size_t i0 = 0; i0 < total; i0 += CH) {
    const size_t n = std::min((size_t)CH, total - i0);
    for (size_t i = 0; i < n; i += 2) {
      const size_t e = i0 + i;
      const int p = (int)(e / d), j = (int)(e % d) / 2;
      const double ang = (double)p * std::pow(base, -2.0 * j / d);
      buf[i] = (float)std::cos(ang);
      buf[i + 1] = (float)std::sin(ang);
    }
    if (hipMemcpy(dst + i0 * 4, buf, n * 4, hipMemcpyHostToDevice) != hipSuccess) return false;
  }
  return true;
}

// The layer descriptor of w[l] / kv[l], validated; PLD_E_INVALID for a missing or misaligned pointer.
pld_status build_layer(const pld_config* cfg, const pld_layer_weights& L, const pld_kv_cache& C, DLayer* out) {
  const bool fp8 = cfg->wfmt == PLD_WFMT_FP8_BLOCK128;
  const bool moe = cfg->ffn_kind == PLD_FFN_MOE;
  const int H = cfg->hidden;
  DLayer& d = *out;
  memset(&d, 0, sizeof(d));
  if (!L.attn_norm || !L.ffn_norm || !aligned16(L.attn_norm) || !aligned16(L.ffn_norm)) return PLD_E_INVALID;
  d.attn_norm = L.attn_norm;
  d.ffn_norm = L.ffn_norm;
  const bool mla = cfg->attn_kind == PLD_ATTN_MLA;
  const bool kda = cfg->attn_kind == PLD_ATTN_KDA;
  if (kda) {
    const int QD = cfg->n_heads * cfg->head_dim, R = cfg->kda_rank;
    if (!mat_ok(L.wq, fp8) || !mat_ok(L.wk, fp8) || !mat_ok(L.wv, fp8) || !mat_ok(L.wo, fp8) || !mat_ok(L.w_g, fp8) ||
        !mat_ok(L.w_beta, fp8) || !mat_ok(L.w_adown, fp8) || !mat_ok(L.w_aup, fp8))
      return PLD_E_INVALID;
    if (!L.conv_taps || !L.o_norm || !aligned16(L.conv_taps) || !aligned16(L.o_norm)) return PLD_E_INVALID;
    d.wq = dmat(L.wq, QD, H, fp8);
    d.wk = dmat(L.wk, QD, H, fp8);
    d.wv = dmat(L.wv, QD, H, fp8);
    d.wo = dmat(L.wo, H, QD, fp8);
    d.w_g = dmat(L.w_g, QD, H, fp8);
    d.w_beta = dmat(L.w_beta, cfg->n_heads, H, fp8);
    d.w_adown = dmat(L.w_adown, R, H, fp8);
    d.w_aup = dmat(L.w_aup, QD, R, fp8);
    d.conv_taps = L.conv_taps;
    d.o_norm = L.o_norm;
  } else if (!mla) {
    const int hd = cfg->head_dim;
    if (!mat_ok(L.wq, fp8) || !mat_ok(L.wk, fp8) || !mat_ok(L.wv, fp8) || !mat_ok(L.wo, fp8)) return PLD_E_INVALID;
    d.wq = dmat(L.wq, cfg->n_heads * hd, H, fp8);
    d.wk = dmat(L.wk, cfg->n_kv_heads * hd, H, fp8);
    d.wv = dmat(L.wv, cfg->n_kv_heads * hd, H, fp8);
    d.wo = dmat(L.wo, H, cfg->n_heads * hd, fp8);
  } else {
    const int NH = cfg->n_heads, QL = cfg->q_lora, KL = cfg->kv_lora, RD = cfg->rope_dim, ND = cfg->nope_dim,
              VD = cfg->v_dim;
    if (!mat_ok(L.w_dq, fp8) || !mat_ok(L.w_uq, fp8) || !mat_ok(L.w_dkv, fp8) || !mat_ok(L.w_uk, fp8) ||
        !mat_ok(L.w_uv, fp8) || !mat_ok(L.wo, fp8))
      return PLD_E_INVALID;
    if (!L.q_norm || !L.kv_norm || !aligned16(L.q_norm) || !aligned16(L.kv_norm)) return PLD_E_INVALID;
    d.q_norm = L.q_norm;
    d.kv_norm = L.kv_norm;
    d.w_dq = dmat(L.w_dq, QL, H, fp8);
    d.w_uq = dmat(L.w_uq, NH * (ND + RD), QL, fp8);
    d.w_dkv = dmat(L.w_dkv, KL + RD, H, fp8);
    d.w_uk = dmat(L.w_uk, NH * ND, KL, fp8);
    d.w_uv = dmat(L.w_uv, NH * VD, KL, fp8);
    d.wo = dmat(L.wo, H, NH * VD, fp8);
    if (cfg->index_topk > 0) {
      const int IH = cfg->index_heads, ID = cfg->index_dim;
      if (!mat_ok(L.w_qi, fp8) || !mat_ok(L.w_w, false) || !mat_ok(L.w_ki, fp8)) return PLD_E_INVALID;
      d.w_qi = dmat(L.w_qi, IH * ID, QL, fp8);
      d.w_w = dmat(L.w_w, IH, H, false);
      d.w_ki = dmat(L.w_ki, ID, H, fp8);
    }
  }
  const bool lutx = cfg->expert_wfmt == PLD_WFMT_LUT3;   // codebooks are required like FP8 scales
  if (!mat_ok(L.w_gate, fp8 || lutx) || !mat_ok(L.w_up, fp8 || lutx) || !mat_ok(L.w_down, fp8 || lutx))
    return PLD_E_INVALID;
  d.w_gate = dmat(L.w_gate, cfg->inter, H, fp8 || lutx);
  d.w_up = dmat(L.w_up, cfg->inter, H, fp8 || lutx);
  d.w_down = dmat(L.w_down, H, cfg->inter, fp8 || lutx);
  if (lutx) {
    d.gu_slot_bytes = (size_t)cfg->inter * H * 3 / 8;
    d.dn_slot_bytes = (size_t)H * cfg->inter * 3 / 8;
    d.gu_slot_cb = (size_t)(cfg->inter / 8) * (H / 64) * 8;
    d.dn_slot_cb = (size_t)(H / 8) * (cfg->inter / 64) * 8;
  } else {
    const size_t wb = fp8 ? 1 : 2;
    d.gu_slot_bytes = (size_t)cfg->inter * H * wb;
    d.dn_slot_bytes = (size_t)H * cfg->inter * wb;
    d.gu_slot_scales = fp8 ? (size_t)((cfg->inter + 127) / 128) * ((H + 127) / 128) : 0;
    d.dn_slot_scales = fp8 ? (size_t)((H + 127) / 128) * ((cfg->inter + 127) / 128) : 0;
  }
  if (moe) {
    if (!L.router || !aligned16(L.router)) return PLD_E_INVALID;
    d.router = (const uint16_t*)L.router;
    if (cfg->router_kind == PLD_ROUTER_SIGMOID_BIAS) {
      if (!L.router_bias) return PLD_E_INVALID;
      d.router_bias = L.router_bias;
    }
  }
  if (kda) {
    if (!C.kda_state || !C.conv_ring || !aligned16(C.kda_state) || !aligned16(C.conv_ring)) return PLD_E_INVALID;
    d.kstate = C.kda_state;
    d.conv_ring = C.conv_ring;
  } else if (!mla) {
    if (!C.k || !C.v || !aligned16(C.k) || !aligned16(C.v)) return PLD_E_INVALID;
    d.kc = (uint16_t*)C.k;
    d.vc = (uint16_t*)C.v;
  } else {
    if (!C.latent || !aligned16(C.latent)) return PLD_E_INVALID;
    d.lat = (uint16_t*)C.latent;
    if (cfg->index_topk > 0) {
      if (!C.index_codes || !C.index_scales || !aligned16(C.index_codes) || !aligned16(C.index_scales))
        return PLD_E_INVALID;
      d.icodes = (uint8_t*)C.index_codes;
      d.iscales = C.index_scales;
    }
  }
  return PLD_OK;
}

// Validates the arguments and fills *h (caller-provided storage) for the workspace `ws`:
// descriptors and the RoPE table uploaded, status and LL buffers zeroed, co-residency
// checked. Allocates nothing, on the host or the device.
pld_status init_into(pld_handle* h, const pld_config* cfg, int32_t n_layers, const pld_layer_weights* w,
                     const pld_kv_cache* kv, const pld_head_weights* head, void* workspace, size_t ws_bytes) {
  if (!cfg || !w || !kv || !workspace || n_layers < 1) return PLD_E_INVALID;
  if (!aligned16(workspace)) return PLD_E_INVALID;
  int dev = 0;
  const int nwg = device_cus(&dev);
  if (nwg <= 0) return PLD_E_HIP;
  KCfg k;
  pld_status st = derive(cfg, nwg, &k);
  if (st != PLD_OK) return st;
  if ((cfg->vocab > 0) != (head != nullptr)) return PLD_E_INVALID;
  if (head && (!head->embed || !head->final_norm || !aligned16(head->embed) || !aligned16(head->final_norm) ||
               !mat_ok(head->head, true)))
    return PLD_E_INVALID;
  const WsOff off = layout(k, n_layers);
  if (ws_bytes < off.total) return PLD_E_CAPACITY;
  uint8_t* ws = (uint8_t*)workspace;
  for (int l = 0; l < n_layers; l++) {   // validate every layer before anything is written
    DLayer d;
    if ((st = build_layer(cfg, w[l], kv[l], &d)) != PLD_OK) return st;
  }
  memset(h, 0, sizeof(*h));
  h->cfg = *cfg;
  h->kc = k;
  h->off = off;
  h->n_layers = n_layers;
  h->ws = ws;
  h->ws_bytes = ws_bytes;
  h->lds_bytes = lds_bytes_for(k.act_floats, k.stage_words, k.outb_floats);
  h->device = dev;
  h->embed = head ? (const uint16_t*)head->embed : nullptr;
  h->fnorm = head ? head->final_norm : nullptr;
  if (head) h->head = dmat(head->head, cfg->vocab, cfg->hidden, true);
  const char* coop = getenv("PLD_COOPERATIVE");
  h->coop = coop && atoi(coop) != 0;
  h->fn = pick_kernel(cfg);
  h->vfn = k.vq >= 2 ? pick_verify(cfg) : nullptr;
  h->bfn = h->vfn ? pick_verify(cfg, true) : nullptr;
  h->vlds_bytes = vlds_bytes();
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) khz = 100000;
  h->wallclock_khz = khz;
  h->budget = (long long)khz * 1000LL * 2;   // 2 s
  bool ok = upload_rope(ws + off.rope, cfg->max_seq, k.rdim, cfg->rope_base);
  for (int l = 0; ok && l < n_layers; l++) {
    DLayer d;
    build_layer(cfg, w[l], kv[l], &d);
    ok = hipMemcpy(ws + off.layers + (size_t)l * sizeof(DLayer), &d, sizeof(DLayer), hipMemcpyHostToDevice) == hipSuccess;
  }
  ok = ok && hipMemset(ws, 0, off.ll_end) == hipSuccess;   // status + LL buffers
  ok = ok && hipFuncSetAttribute((const void*)h->fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)h->lds_bytes) == hipSuccess;
  int per_cu = 0;
  ok = ok && hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)h->fn, BLOCK, h->lds_bytes) == hipSuccess;
  for (KernelFn f : {h->vfn, h->bfn}) {
    if (!ok || !f) continue;
    int per_v = 0;
    ok = hipFuncSetAttribute((const void*)f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)h->vlds_bytes) ==
             hipSuccess &&
         hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_v, (const void*)f, BLOCK, h->vlds_bytes) == hipSuccess;
    per_cu = std::min(per_cu, per_v);
  }
  ok = ok && hipDeviceSynchronize() == hipSuccess;
  if (!ok) return PLD_E_HIP;
  if (per_cu < 1) return PLD_E_UNSUPPORTED;
  return PLD_OK;
}

constexpr size_t STATIC_WS_BYTES = (size_t)32 << 20;
constexpr int MAX_DEVICES = 64;
void* scratch_dev[MAX_DEVICES];         // device address of `scratch` on each device, once looked up
pld_handle static_handle[MAX_DEVICES];  // the handle decode_layer_init_static returns on each device

}  // namespace

// Workspace of decode_layer_init_static (no allocation): 32 MiB that every device the library
// runs on holds until the process ends. In host code `scratch` names a host-side stand-in;
// its device address on the current device comes from hipGetSymbolAddress (scratch_dev[]).
static __device__ __align__(256) uint8_t scratch[STATIC_WS_BYTES];

extern "C" {

pld_status decode_layer_init(const pld_config* cfg, int32_t n_layers, const pld_layer_weights* w,
                             const pld_kv_cache* kv, const pld_head_weights* head, void* workspace, size_t ws_bytes,
                             pld_handle** out) {
  if (!out) return PLD_E_INVALID;
  *out = nullptr;
  pld_handle* h = new (std::nothrow) pld_handle();
  if (!h) return PLD_E_INVALID;
  const pld_status st = init_into(h, cfg, n_layers, w, kv, head, workspace, ws_bytes);
  if (st != PLD_OK) {
    delete h;
    return st;
  }
  *out = h;
  return PLD_OK;
}

pld_status decode_layer_init_static(const pld_config* cfg, int32_t n_layers, const pld_layer_weights* w,
                                    const pld_kv_cache* kv, const pld_head_weights* head, pld_handle** out) {
  if (!out) return PLD_E_INVALID;
  *out = nullptr;
  if (!cfg || n_layers < 1) return PLD_E_INVALID;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PLD_E_HIP;
  if (dev < 0 || dev >= MAX_DEVICES) return PLD_E_UNSUPPORTED;
  if (!scratch_dev[dev]) {   // once per device, with that device current
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PLD_E_HIP;
    scratch_dev[dev] = p;
  }
  const int nwg = device_cus(nullptr);
  if (nwg <= 0) return PLD_E_HIP;
  KCfg k;
  const pld_status sd = derive(cfg, nwg, &k);
  if (sd != PLD_OK) return sd;
  if (layout(k, n_layers).total > STATIC_WS_BYTES) return PLD_E_CAPACITY;
  pld_handle* h = &static_handle[dev];
  const uint32_t steps = h->steps;   // the LL epoch keeps counting across re-initialisations
  const pld_status st = init_into(h, cfg, n_layers, w, kv, head, scratch_dev[dev], STATIC_WS_BYTES);
  h->steps = steps;
  h->is_static = true;
  if (st != PLD_OK) return st;
  *out = h;
  return PLD_OK;
}

struct HeadArgs {
  int on, in_token;
  float* out_logits;
  int32_t* out_tokens;
  const int32_t* drafts;
  int32_t* out_accepted;
  double temperature;
  uint64_t sample_seed;
};

static pld_status launch(pld_handle* h, int layer0, int n_layers, int n_tokens, int pos0, const void* in_hidden,
                         void* out_hidden, hipStream_t s, HeadArgs hd = {0, -1, nullptr, nullptr, nullptr, nullptr, 0.0, 0}) {
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
  a.head_on = hd.on;
  a.in_token = hd.in_token;
  a.out_logits = hd.out_logits;
  a.out_tokens = hd.out_tokens;
  a.drafts = hd.drafts;
  a.out_accepted = hd.out_accepted;
  a.embed = h->embed;
  a.fnorm = h->fnorm;
  a.head = h->head;
  a.hooks = h->hooks;
  a.hook_seed = h->hook_seed;
  a.temperature = hd.temperature;
  a.sample_seed = hd.sample_seed;
  hipError_t e;
  if (h->coop) {
    void* args[] = {&a};
    e = hipLaunchCooperativeKernel((const void*)h->fn, dim3(h->kc.nwg), dim3(BLOCK), args, (unsigned)h->lds_bytes, s);
  } else {
    void* args[] = {&a};
    e = hipLaunchKernel((const void*)h->fn, dim3(h->kc.nwg), dim3(BLOCK), args, h->lds_bytes, s);
  }
  if (e != hipSuccess) return PLD_E_HIP;
  h->hooks &= ~PLD_HOOK_DROP_WG0;   // lasts one launch
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
  const bool head = h->cfg.vocab > 0;
  if (a->n_tokens < 1 || a->n_query < 1) return PLD_E_INVALID;
  const bool verify = a->n_query > 1;
  if (verify) {
    // n_query positions start_pos.. fed in_token then the n_query - 1 drafts; one verify per launch
    if (!head) return PLD_E_UNSUPPORTED;
    if (a->n_tokens != 1 || a->in_token < 0 || !a->draft_tokens || ((uintptr_t)a->draft_tokens & 3u))
      return PLD_E_INVALID;
  } else if (a->draft_tokens || a->out_accepted) {
    return PLD_E_INVALID;
  }
  const int n_pos = verify ? a->n_query : a->n_tokens;
  if (!head && (a->in_token >= 0 || a->n_tokens != 1 || a->out_logits || a->out_tokens))
    return PLD_E_INVALID;   // embedding input, several tokens and logits/tokens need the LM head
  if (a->in_token >= h->cfg.vocab && head) return PLD_E_INVALID;
  if (a->in_token < 0 && (!a->in_hidden || !aligned16(a->in_hidden))) return PLD_E_INVALID;
  if (!a->out_hidden || !aligned16(a->out_hidden)) return PLD_E_INVALID;
  if (a->start_pos < 0 || a->start_pos + n_pos > h->cfg.max_seq) return PLD_E_CAPACITY;
  if (!(a->temperature >= 0.0) || !std::isfinite(a->temperature) || (a->temperature > 0.0 && !head))
    return PLD_E_INVALID;
  HeadArgs hd{head ? 1 : 0, head ? a->in_token : -1, a->out_logits, a->out_tokens,
              verify ? a->draft_tokens : nullptr, verify ? a->out_accepted : nullptr, a->temperature,
              a->sample_seed};
  return launch(h, 0, h->n_layers, n_pos, a->start_pos, a->in_token >= 0 ? nullptr : a->in_hidden, a->out_hidden,
                (hipStream_t)stream, hd);
}

pld_status decode_verify_batched(pld_handle* h, const pld_persistent_args* a, void* stream) {
  if (!h || !a) return PLD_E_INVALID;
  if (h->bad) return PLD_E_STATE;
  if (!h->vfn || h->cfg.max_query < 2) return PLD_E_UNSUPPORTED;
  const int nq = a->n_query;
  if (nq < 2 || nq > h->cfg.max_query || a->n_tokens != 1) return PLD_E_INVALID;
  if (a->in_token < 0 || a->in_token >= h->cfg.vocab || !a->draft_tokens || ((uintptr_t)a->draft_tokens & 3u))
    return PLD_E_INVALID;
  if (!a->out_hidden || !aligned16(a->out_hidden)) return PLD_E_INVALID;
  if (a->start_pos < 0 || a->start_pos + nq > h->cfg.max_seq) return PLD_E_CAPACITY;
  if (!(a->temperature >= 0.0) || !std::isfinite(a->temperature)) return PLD_E_INVALID;
  KArgs k;
  memset(&k, 0, sizeof(k));
  k.c = h->kc;
  k.ws = h->ws;
  k.off = h->off;
  k.n_layers = h->n_layers;
  k.n_tokens = 1;
  k.nrows = nq;
  k.bmode = 0;
  k.pos0 = a->start_pos;
  k.layer0 = 0;
  k.step0 = h->steps;
  k.out_hidden = (uint16_t*)a->out_hidden;
  k.budget = h->budget;
  k.trace = h->trace;
  k.trace_steps = h->trace_steps;
  k.head_on = 1;
  k.in_token = a->in_token;
  k.out_logits = a->out_logits;
  k.out_tokens = a->out_tokens;
  k.drafts = a->draft_tokens;
  k.out_accepted = a->out_accepted;
  k.embed = h->embed;
  k.fnorm = h->fnorm;
  k.head = h->head;
  k.hooks = h->hooks;
  k.hook_seed = h->hook_seed;
  k.temperature = a->temperature;
  k.sample_seed = a->sample_seed;
  void* args[] = {&k};
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = h->coop ? hipLaunchCooperativeKernel((const void*)h->vfn, dim3(h->kc.nwg), dim3(BLOCK), args,
                                                            (unsigned)h->vlds_bytes, s)
                               : hipLaunchKernel((const void*)h->vfn, dim3(h->kc.nwg), dim3(BLOCK), args, h->vlds_bytes, s);
  if (e != hipSuccess) return PLD_E_HIP;
  h->hooks &= ~PLD_HOOK_DROP_WG0;
  h->steps += (uint32_t)h->n_layers;
  h->last_stream = s;
  return PLD_OK;
}

pld_status decode_batch(pld_handle* h, const pld_batch_args* a, void* stream) {
  if (!h || !a) return PLD_E_INVALID;
  if (h->bad) return PLD_E_STATE;
  if (!h->bfn || h->kc.vb < 2) return PLD_E_UNSUPPORTED;
  const int nb = a->n_seq;
  if (nb < 2 || nb > h->kc.vb || a->n_tokens < 1) return PLD_E_INVALID;
  if (!a->out_tokens || ((uintptr_t)a->out_tokens & 3u) || !a->out_hidden || !aligned16(a->out_hidden))
    return PLD_E_INVALID;
  if (!(a->temperature >= 0.0) || !std::isfinite(a->temperature)) return PLD_E_INVALID;
  for (int b = 0; b < nb; b++) {
    if (a->in_token[b] < 0 || a->in_token[b] >= h->cfg.vocab) return PLD_E_INVALID;
    if (a->start_pos[b] < 0 || (long long)a->start_pos[b] + a->n_tokens > h->cfg.max_seq) return PLD_E_CAPACITY;
  }
  if ((long long)a->n_tokens * h->n_layers > (1ll << 24)) return PLD_E_INVALID;
  KArgs k;
  memset(&k, 0, sizeof(k));
  k.c = h->kc;
  k.ws = h->ws;
  k.off = h->off;
  k.n_layers = h->n_layers;
  k.n_tokens = a->n_tokens;
  k.nrows = nb;
  k.bmode = 1;
  for (int b = 0; b < nb; b++) {
    k.bpos[b] = a->start_pos[b];
    k.btok[b] = a->in_token[b];
  }
  k.pos0 = a->start_pos[0];
  k.layer0 = 0;
  k.step0 = h->steps;
  k.out_hidden = (uint16_t*)a->out_hidden;
  k.budget = h->budget;
  k.trace = h->trace;
  k.trace_steps = h->trace_steps;
  k.head_on = 1;
  k.in_token = a->in_token[0];
  k.out_logits = a->out_logits;
  k.out_tokens = a->out_tokens;
  k.embed = h->embed;
  k.fnorm = h->fnorm;
  k.head = h->head;
  k.hooks = h->hooks;
  k.hook_seed = h->hook_seed;
  k.temperature = a->temperature;
  k.sample_seed = a->sample_seed;
  void* args[] = {&k};
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = h->coop ? hipLaunchCooperativeKernel((const void*)h->bfn, dim3(h->kc.nwg), dim3(BLOCK), args,
                                                            (unsigned)h->vlds_bytes, s)
                               : hipLaunchKernel((const void*)h->bfn, dim3(h->kc.nwg), dim3(BLOCK), args, h->vlds_bytes, s);
  if (e != hipSuccess) return PLD_E_HIP;
  h->hooks &= ~PLD_HOOK_DROP_WG0;
  h->steps += (uint32_t)(h->n_layers * a->n_tokens);
  h->last_stream = s;
  return PLD_OK;
}

pld_status decode_poll_status(pld_handle* h, pld_device_status* out) {
  if (!h || !out) return PLD_E_INVALID;
  int32_t st[8];
  if (hipStreamSynchronize(h->last_stream) != hipSuccess) return PLD_E_HIP;
  if (hipMemcpyAsync(st, h->ws + h->off.status, sizeof(st), hipMemcpyDeviceToHost, h->last_stream) != hipSuccess ||
      hipStreamSynchronize(h->last_stream) != hipSuccess)
    return PLD_E_HIP;
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
  // status and LL buffers cleared on the handle's stream; the step counter (LL epoch) keeps
  // counting, so no word left by an aborted launch can carry an epoch that a later launch waits for
  if (hipStreamSynchronize(h->last_stream) != hipSuccess) return PLD_E_HIP;
  if (hipMemsetAsync(h->ws, 0, h->off.ll_end, h->last_stream) != hipSuccess) return PLD_E_HIP;
  if (hipStreamSynchronize(h->last_stream) != hipSuccess) return PLD_E_HIP;
  h->bad = false;
  return PLD_OK;
}

void decode_layer_destroy(pld_handle* h) {
  if (h && !h->is_static) delete h;
}

pld_status pld_set_test_hooks(pld_handle* h, int32_t flags, uint32_t seed) {
  if (!h || (flags & ~(PLD_HOOK_DROP_WG0 | PLD_HOOK_DELAY))) return PLD_E_INVALID;
  h->hooks = flags;
  h->hook_seed = seed;
  return PLD_OK;
}

// Host loop of speculative decoding over two handles that share the LM head and
// embedding: the draft stack proposes n_draft tokens from the current position (one launch),
// the target verifies them in one launch, the accepted drafts and the target's token after
// them are kept, and both continue after the last kept token. Invariant at the top of the
// loop: both caches hold correct rows for every position < p, and t is the (kept) token at p.
// A verify writes target rows p .. p+nd (inputs t, d_0 .. d_{nd-1}); the draft launch wrote
// draft rows p .. p+nd-1 (inputs t, d_0 .. d_{nd-2}); keeping m drafts needs rows up to p+m,
// so only m == nd needs one more draft step (input d_{nd-1} at p+nd).
pld_status decode_speculative(pld_handle* target, pld_handle* draft, const pld_spec_args* a, void* stream) {
  if (!target || !draft || !a || !a->out_tokens || ((uintptr_t)a->out_tokens & 3u)) return PLD_E_INVALID;
  if (target->bad || draft->bad) return PLD_E_STATE;
  if (target->cfg.vocab <= 0 || draft->cfg.vocab != target->cfg.vocab || draft->embed != target->embed ||
      draft->head.w != target->head.w)
    return PLD_E_INVALID;   // the two stacks must share the vocabulary, embedding and head
  if (a->n_tokens < 1 || a->n_draft < 1 || a->n_draft > 15 || a->in_token < 0 || a->in_token >= target->cfg.vocab)
    return PLD_E_INVALID;
  if (!(a->temperature >= 0.0) || !std::isfinite(a->temperature)) return PLD_E_INVALID;
  const int last_pos = a->start_pos + a->n_tokens;   // no launch writes a row beyond this
  if (a->start_pos < 0 || last_pos > target->cfg.max_seq || last_pos > draft->cfg.max_seq) return PLD_E_CAPACITY;
  hipStream_t s = (hipStream_t)stream;
  int32_t* sp = (int32_t*)(target->ws + target->off.spec);
  int32_t* d_drafts = sp;            // [16]
  int32_t* d_vtok = sp + 16;         // [16]
  int32_t* d_acc = sp + 32;          // [1]
  int32_t* d_junk = sp + 33;         // [1] output of a catch-up draft step
  int p = a->start_pos, t = a->in_token, produced = 0, verifies = 0, acc_total = 0;
  HeadArgs hd{1, 0, nullptr, nullptr, nullptr, nullptr, a->temperature, a->sample_seed};
  pld_status st;
  while (produced < a->n_tokens) {
    const int remaining = a->n_tokens - produced;
    if (remaining == 1) {   // one token left: a plain target step
      HeadArgs h1 = hd;
      h1.in_token = t;
      h1.out_tokens = a->out_tokens + produced;
      if ((st = launch(target, 0, target->n_layers, 1, p, nullptr, nullptr, s, h1)) != PLD_OK)
        return st;
      produced += 1;
      break;
    }
    const int nd = std::min(a->n_draft, remaining - 1);
    HeadArgs hdr = hd;
    hdr.in_token = t;
    hdr.out_tokens = d_drafts;
    if ((st = launch(draft, 0, draft->n_layers, nd, p, nullptr, nullptr, s, hdr)) != PLD_OK)
      return st;
    HeadArgs hv = hd;
    hv.in_token = t;
    hv.out_tokens = d_vtok;
    hv.drafts = d_drafts;
    hv.out_accepted = d_acc;
    if ((st = launch(target, 0, target->n_layers, nd + 1, p, nullptr, nullptr, s, hv)) != PLD_OK)
      return st;
    verifies++;
    int32_t host[17];
    if (hipMemcpyAsync(host, d_vtok, 17 * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return PLD_E_HIP;
    const int m = host[16];
    if (m < 0 || m > nd) return PLD_E_HIP;
    const int keep = std::min(m + 1, remaining);
    if (hipMemcpyAsync(a->out_tokens + produced, d_vtok, keep * sizeof(int32_t), hipMemcpyDeviceToDevice, s) !=
        hipSuccess)
      return PLD_E_HIP;
    produced += keep;
    acc_total += m;
    if (m == nd && produced < a->n_tokens) {   // the draft cache lacks the row of its last draft
      HeadArgs hc = hd;
      hc.in_token = host[nd - 1];
      hc.out_tokens = d_junk;
      if ((st = launch(draft, 0, draft->n_layers, 1, p + nd, nullptr, nullptr, s, hc)) != PLD_OK)
        return st;
    }
    p += m + 1;
    t = host[m];
  }
  if (a->out_stats) {
    a->out_stats[0] = verifies;
    a->out_stats[1] = acc_total;
  }
  return PLD_OK;
}

pld_status pld_debug_buffer(pld_handle* h, const char* name, void** ptr, size_t* bytes) {
  if (!h || !name || !ptr || !bytes) return PLD_E_INVALID;
  const KCfg& k = h->kc;
  struct E { const char* n; size_t off, sz; } tab[] = {
      {"a", h->off.a_dbg, (size_t)k.H * 4},
      {"q", h->off.q, (size_t)k.nh * (k.attn == PLD_ATTN_MLA ? k.nope : k.hd) * 8},
      {"o", h->off.o, (size_t)k.nh * (k.attn == PLD_ATTN_MLA ? k.vdim : k.hd) * 8},
      {"h2", h->off.h2, (size_t)k.H * 8},
      {"b", h->off.b_dbg, (size_t)k.H * 4},
      {"f", h->off.f_dbg, (size_t)k.H * 4},
      {"logits", h->off.logits, (size_t)k.E * 32},
      {"sel", h->off.sel, (size_t)k.topk * 4},
      {"gates", h->off.gates, (size_t)k.topk * 4},
      {"m", h->off.m, (size_t)k.slots * k.inter * 8},
      {"x", h->off.x, (size_t)k.H * 4},
      {"cq", h->off.cqr, (size_t)k.q_lora * (k.itopk > 0 ? 2 : 1) * 8},
      {"ckv", h->off.ckvr, (size_t)(k.kv_lora + k.rope) * 8},
      {"qrope", h->off.qr, (size_t)k.nh * k.rope * 8},
      {"qlat", h->off.qlat, (size_t)k.nh * k.kv_lora * 8},
      {"olat", h->off.olat, (size_t)k.nh * k.kv_lora * 8},
      {"qi", h->off.qi, (size_t)k.ih * k.idim / 2 * 8},
      {"ixr", h->off.ixr, (size_t)(k.ih + k.idim) * 8},
      {"isel", h->off.isel, (size_t)k.itopk * 8},
      {"ikh", h->off.ikh, (size_t)k.max_seq * 4},
      {"ikl", h->off.ikl, (size_t)k.max_seq * 4},
      {"ilist", h->off.ilist, (size_t)k.nwg * SEL_LIST * 8},
      {"ilo", h->off.ilo, (size_t)k.nwg * SEL_LIST * 4},
      {"itok", h->off.itok, (size_t)k.nwg * SEL_LIST * 4},
      {"part", h->off.part, k.attn == PLD_ATTN_MLA ? (size_t)k.nh * k.cpg * (k.kv_lora + 2) * 8
                                                    : (size_t)k.nh * k.cpg * (k.hd + 2) * 8},
      {"kv", h->off.kv, (size_t)std::max(k.nkv * k.hd, 1) * 8},
      {"amax", h->off.amax, (size_t)3 * std::max(k.nwg, 1) * 8},
      // batched verify (handles made with max_query >= 2): per-position LL buffers, 8 positions
      {"vx", h->off.vx, k.vq >= 2 ? (size_t)8 * (k.H / 2) * 8 : 0},
      {"vcq", h->off.vcqr, k.vq >= 2 ? (size_t)8 * k.q_lora * 8 : 0},
      {"vckv", h->off.vckv, k.vq >= 2 ? (size_t)8 * (k.kv_lora + k.rope) * 8 : 0},
      {"vqlat", h->off.vqlat, k.vq >= 2 ? (size_t)8 * (k.nh * k.kv_lora / 2) * 8 : 0},
      {"volat", h->off.volat, k.vq >= 2 ? (size_t)8 * k.nh * k.kv_lora * 8 : 0},
      {"vo", h->off.vo, k.vq >= 2 ? (size_t)8 * (k.nh * k.vdim / 2) * 8 : 0},
      {"vh2", h->off.vh2, k.vq >= 2 ? (size_t)8 * k.H * 8 : 0},
      {"vsel", h->off.vsel, k.vq >= 2 ? (size_t)8 * 8 * 4 * 2 : 0},
      {"vf", h->off.vf, k.vq >= 2 ? (size_t)8 * k.H * 4 : 0},
  };
  for (auto& e : tab)
    if (!strcmp(e.n, name)) {
      if (e.sz == 0) return PLD_E_INVALID;
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
