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
enum Stage { S_QKV = 0, S_H2 = 1, S_RT = 2, S_M = 3, S_OUT = 4, NSTG = 8 };
enum { ST_CODE = 0, ST_STAGE = 1, ST_LAYER = 2, ST_TOKEN = 3, ST_WG = 4, ST_ABORT = 8 };

struct KCfg {
  int attn, wfmt, H, nh, nkv, hd, q_lora, kv_lora, rope, nope, vdim, ih, idim, itopk;
  int ffn, inter, E, topk, nshared, router, max_seq, vocab;
  double eps;
  int slots;   // expert slots used per token (routed + shared), 1 for a dense FFN
  int G;       // q heads per kv head
  int cpg;     // attention chunks per kv head = workgroups per kv head
  int chmax;   // max tokens in one attention chunk
  int act_floats, outb_floats;
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

// Hidden-state source: the caller's bf16 input, or the in-launch buffer of bf16 words.
struct XSrc {
  const uint16_t* p16;
  const uint32_t* p32;
  __device__ __forceinline__ float operator()(int i) const {
    return p32 ? __uint_as_float(ld_u32(p32 + i) << 16) : bf16_to_f32(gp(p16)[i]);
  }
};

// act[i] = fp32((x_i * r) * g_i), r = 1/sqrt(sum(x^2)/n + eps), statistics in fp64.
template <typename LoadX>
__device__ __forceinline__ void rmsnorm_to_lds(LoadX ldx, const float* __restrict__ gamma, int n, double eps, float* act, double* red) {
  double ss = 0.0;
  for (int i = threadIdx.x; i < n; i += BLOCK) {
    const float v = ldx(i);
    act[i] = v;
    ss += (double)v * (double)v;
  }
  ss = block_sum(ss, red);
  const double r = 1.0 / sqrt(ss / (double)n + eps);
  for (int i = threadIdx.x; i < n; i += BLOCK) act[i] = (float)(((double)act[i] * r) * (double)gp(gamma)[i]);
  __syncthreads();
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// ------------------------------------------------------------------ top-k (one wave)
// Selects k of n fp64 scores (desc, lowest index on ties); writes indices in selection order.
__device__ void wave_topk(const double* score, int n, int k, int* sel_out) {
  const int lane = threadIdx.x & 63;
  constexpr int PER = 8;   // up to 512 candidates
  double v[PER];
  int id[PER];
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int e = lane + 64 * i;
    v[i] = e < n ? score[e] : -INFINITY;
    id[i] = e < n ? e : 0x7fffffff;
  }
  for (int s = 0; s < k; s++) {
    double bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < PER; i++)
      if (v[i] > bv || (v[i] == bv && id[i] < bi)) { bv = v[i]; bi = id[i]; }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) sel_out[s] = bi;
#pragma unroll
    for (int i = 0; i < PER; i++)
      if (id[i] == bi) { v[i] = -INFINITY; id[i] = 0x7fffffff; }
  }
}

// ------------------------------------------------------------------ LDS layout
struct Lds {
  float* act;   // [act_floats]
  float* outb;  // [outb_floats]
  float* outc;  // [outb_floats]
  double* red;  // [16]
  int* isel;    // [32]
  float* fgate; // [32]
  int* flag;    // [8]
};
__device__ __forceinline__ Lds carve(float* base, const KCfg& c) {
  Lds L;
  L.act = base;
  L.outb = base + c.act_floats;
  L.outc = L.outb + c.outb_floats;
  L.red = reinterpret_cast<double*>(L.outc + c.outb_floats);
  L.isel = reinterpret_cast<int*>(L.red + 16);
  L.fgate = reinterpret_cast<float*>(L.isel + 32);
  L.flag = reinterpret_cast<int*>(L.fgate + 32);
  return L;
}
__host__ __device__ inline size_t lds_bytes_for(int act_floats, int outb_floats) {
  return (size_t)4 * (act_floats + 2 * outb_floats) + 8 * 16 + 4 * 32 + 4 * 32 + 4 * 8;
}

// ------------------------------------------------------------------ compiled layer shapes
// One kernel is compiled per supported layer shape, so every reduction length, head
// size and expert width is a compile-time constant: each GEMV call site gets exactly one
// lane layout, and the whole step inlines into the kernel (no device calls on the hot
// path). Row counts that vary at run time (experts, top-k, cache length) stay runtime.
template <int H_, int NH_, int NKV_, int HD_, int INTER_, bool FP8_, bool MOE_>
struct GqaShape {
  static constexpr int H = H_, NH = NH_, NKV = NKV_, HD = HD_, INTER = INTER_;
  static constexpr int G = NH / NKV, ODIM = NH * HD;
  static constexpr bool FP8 = FP8_, MOE = MOE_;
};

// Per-(token, layer) state of one workgroup.
struct Step {
  const DLayer* Ly;
  XSrc xs;
  uint32_t k1;   // step number + 1 (counter epoch)
  bool first;    // first step of the launch: input comes from the caller
  int pos;
};

template <bool FP8, int K, typename Pre>
__device__ __forceinline__ bool mv(const DMat& M, size_t boff, size_t soff, int r0, int r1, const float* act,
                                   float* out, int mode, float alpha, Pre&& pre) {
  return gemv<FP8, K, float>(M.w + boff, FP8 ? M.s + soff : nullptr, r0, r1, act, out, mode, alpha, pre);
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
  bool pending = true;   // the input wait + RMSNorm has not run yet
  auto pre_x = [&]() -> bool {
    if (!pending) return true;
    pending = false;
    if (!st.first && !wait_all(cx, S_OUT, st.k1 - 1, nwg)) return false;
    rmsnorm_to_lds(st.xs, Ly.attn_norm, SH::H, c.eps, L.act, L.red);
    if (w == 0)
      for (int i = threadIdx.x; i < SH::H; i += BLOCK) st_f32(wsp<float>(a, a.off.a_dbg) + i, L.act[i]);
    return true;
  };
  {
    const int lo = max(r0, 0), hi = min(r1, qR);
    if (lo < hi && !mv<SH::FP8, SH::H>(Ly.wq, 0, 0, lo, hi, L.act, L.outb + (lo - r0), OUT_STORE, 1.f, pre_x)) return false;
  }
  {
    const int lo = max(r0, qR), hi = min(r1, qR + kR);
    if (lo < hi && !mv<SH::FP8, SH::H>(Ly.wk, 0, 0, lo - qR, hi - qR, L.act, L.outb + (lo - r0), OUT_STORE, 1.f, pre_x))
      return false;
  }
  {
    const int lo = max(r0, qR + kR), hi = min(r1, R);
    if (lo < hi &&
        !mv<SH::FP8, SH::H>(Ly.wv, 0, 0, lo - qR - kR, hi - qR - kR, L.act, L.outb + (lo - r0), OUT_STORE, 1.f, pre_x))
      return false;
  }
  if (!pre_x()) return false;
  __syncthreads();
  const float* rope = wsp<float>(a, a.off.rope) + (size_t)pos * HD;   // (cos, sin) pairs, HD/2 per position
  float* qw = wsp<float>(a, a.off.q);
  for (int p = r0 / 2 + threadIdx.x; p < r1 / 2; p += BLOCK) {
    const int r = 2 * p;
    float v0 = L.outb[r - r0], v1 = L.outb[r + 1 - r0];
    if (r < qR + kR) {
      const int d = (r < qR ? r : r - qR) % HD;
      const float cs = gp(rope)[d], sn = gp(rope)[d + 1];
      const float x0 = v0 * cs - v1 * sn, x1 = v0 * sn + v1 * cs;
      v0 = x0;
      v1 = x1;
    }
    if (r < qR) {
      st_f32(qw + r, v0);
      st_f32(qw + r + 1, v1);
    } else {
      const bool isk = r < qR + kR;
      const int rr = isk ? r - qR : r - qR - kR;
      const int head = rr / HD, d = rr % HD;
      uint16_t* dst = (isk ? Ly.kc : Ly.vc) + ((size_t)head * c.max_seq + pos) * HD + d;
      st_u32(reinterpret_cast<uint32_t*>(dst), f32_to_bf16(v0) | (f32_to_bf16(v1) << 16));
    }
  }
  arrive(cx, S_QKV, st.k1, nwg);
  return true;
}

// ------------------------------------------------------------------ attention (GQA)
// One workgroup = one (kv head g, token chunk) pair. Scores for the G query heads of
// the group, chunk-local softmax, P.V, then a partial (m, l, acc[HD]) per head. The
// group's last arriver merges the partials into o.
template <class SH>
__device__ __forceinline__ bool attention_gqa(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  const uint32_t k1 = st.k1;
  constexpr int HD = SH::HD, G = SH::G;
  constexpr int LPT = HD / 8;      // lanes per token row (16 bytes each)
  constexpr int TPW = 64 / LPT;    // tokens per wave pass
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int dl = lane % LPT, tl = lane / LPT;
  const int cpg = c.cpg;
  const int g = cx.w / cpg, ch = cx.w % cpg;
  const int T = st.pos + 1;
  const int t0 = split_at(T, cpg, ch), t1 = split_at(T, cpg, ch + 1), n = t1 - t0;
  const uint16_t* kbase = Ly.kc + (size_t)g * c.max_seq * HD;
  const uint16_t* vbase = Ly.vc + (size_t)g * c.max_seq * HD;
  const int fresh = a.pos0;   // rows >= fresh were written inside this launch

  auto load_row = [&](const uint16_t* base, int t) -> uint4 {
    const uint16_t* p = base + (size_t)t * HD + dl * 8;
    if (t >= fresh) {
      const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
      return make_uint4(ld_u32(q), ld_u32(q + 1), ld_u32(q + 2), ld_u32(q + 3));
    }
    return ld_g16(p);
  };

  // static history rows are issued before the wait for this step's q/k/v
  uint4 kpre = make_uint4(0u, 0u, 0u, 0u);
  {
    const int t = wave * TPW + tl;
    if (t < n && t0 + t < fresh) kpre = ld_g16(kbase + (size_t)(t0 + t) * HD + dl * 8);
  }
  if (!wait_all(cx, S_QKV, k1, cx.nwg)) return false;

  const float* qg = wsp<float>(a, a.off.q) + (size_t)g * G * HD;
  const float scale = 1.0f / sqrtf((float)HD);
  float qr[G][8];
#pragma unroll
  for (int h = 0; h < G; h++)
#pragma unroll
    for (int j = 0; j < 8; j++) qr[h][j] = ld_f32(qg + h * HD + dl * 8 + j) * scale;

  float* sc = L.act;                               // [G][chmax]
  float* red2 = L.act + G * c.chmax;               // [NWAVES][G][HD]
  float* ml = red2 + NWAVES * G * HD;              // [2G]
  for (int tb = 0; tb < n; tb += NWAVES * TPW) {
    const int t = tb + wave * TPW + tl;
    float s[G];
#pragma unroll
    for (int h = 0; h < G; h++) s[h] = 0.f;
    if (t < n) {
      const uint4 kv = (tb == 0 && t0 + t < fresh) ? kpre : load_row(kbase, t0 + t);
      float kf[8] = {bf_lo(kv.x), bf_hi(kv.x), bf_lo(kv.y), bf_hi(kv.y), bf_lo(kv.z), bf_hi(kv.z), bf_lo(kv.w), bf_hi(kv.w)};
#pragma unroll
      for (int h = 0; h < G; h++)
#pragma unroll
        for (int j = 0; j < 8; j++) s[h] = fmaf(qr[h][j], kf[j], s[h]);
    }
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
      for (int off = LPT / 2; off >= 1; off >>= 1) s[h] += __shfl_xor(s[h], off, 64);
    if (dl == 0 && t < n)
#pragma unroll
      for (int h = 0; h < G; h++) sc[h * c.chmax + t] = s[h];
  }
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
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; h++)
#pragma unroll
    for (int j = 0; j < 8; j++) acc[h][j] = 0.f;
  for (int tb = 0; tb < n; tb += NWAVES * TPW) {
    const int t = tb + wave * TPW + tl;
    if (t < n) {
      const uint4 vv = load_row(vbase, t0 + t);
      float vf[8] = {bf_lo(vv.x), bf_hi(vv.x), bf_lo(vv.y), bf_hi(vv.y), bf_lo(vv.z), bf_hi(vv.z), bf_lo(vv.w), bf_hi(vv.w)};
#pragma unroll
      for (int h = 0; h < G; h++) {
        const float p = sc[h * c.chmax + t];
#pragma unroll
        for (int j = 0; j < 8; j++) acc[h][j] = fmaf(p, vf[j], acc[h][j]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; h++)
#pragma unroll
    for (int j = 0; j < 8; j++)
#pragma unroll
      for (int off = LPT; off < 64; off <<= 1) acc[h][j] += __shfl_xor(acc[h][j], off, 64);
  if (tl == 0)
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
      for (int j = 0; j < 8; j++) red2[(wave * G + h) * HD + dl * 8 + j] = acc[h][j];
  __syncthreads();
  float* part = wsp<float>(a, a.off.part);
  for (int i = threadIdx.x; i < G * HD; i += BLOCK) {
    float s = 0.f;
#pragma unroll
    for (int wv = 0; wv < NWAVES; wv++) s += red2[wv * G * HD + i];
    const int h = i / HD, d = i % HD;
    st_f32(part + ((size_t)(g * G + h) * cpg + ch) * (HD + 2) + 2 + d, s);
  }
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float* pp = part + ((size_t)(g * G + h) * cpg + ch) * (HD + 2);
    st_f32(pp, ml[2 * h]);
    st_f32(pp + 1, ml[2 * h + 1]);
  }
  // last arriver of the group merges
  vm_wait();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = atomic_add_u32(cx.ctr_grp + g * CTR_STRIDE, 1u);
    L.flag[0] = (old + 1u == k1 * (uint32_t)cpg);
  }
  __syncthreads();
  if (L.flag[0]) {
    float* mlc = L.act;  // [G][cpg][2]
    for (int i = threadIdx.x; i < G * cpg; i += BLOCK) {
      const int h = i / cpg, cc = i % cpg;
      const float* pp = part + ((size_t)(g * G + h) * cpg + cc) * (HD + 2);
      mlc[2 * i] = ld_f32(pp);
      mlc[2 * i + 1] = ld_f32(pp + 1);
    }
    __syncthreads();
    float* obuf = wsp<float>(a, a.off.o);
    for (int i = threadIdx.x; i < G * HD; i += BLOCK) {
      const int h = i / HD, d = i % HD;
      float M = -INFINITY;
      for (int cc = 0; cc < cpg; cc++)
        if (mlc[2 * (h * cpg + cc) + 1] > 0.f) M = fmaxf(M, mlc[2 * (h * cpg + cc)]);
      float Ls = 0.f, o = 0.f;
      for (int cc = 0; cc < cpg; cc++) {
        const float l = mlc[2 * (h * cpg + cc) + 1];
        if (l > 0.f) {
          const float f = __expf(mlc[2 * (h * cpg + cc)] - M);
          Ls += f * l;
          o += f * ld_f32(part + ((size_t)(g * G + h) * cpg + cc) * (HD + 2) + 2 + d);
        }
      }
      st_f32(obuf + (size_t)(g * G + h) * HD + d, o / Ls);
    }
    vm_wait();
    __syncthreads();
    if (threadIdx.x == 0) atomic_add_u32(cx.ctr_att, 1u);
  }
  return true;
}

// ------------------------------------------------------------------ stage: output projection + residual
template <class SH>
__device__ __forceinline__ bool stage_wo(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const int r0 = split_at(SH::H, cx.nwg, cx.w), r1 = split_at(SH::H, cx.nwg, cx.w + 1);
  auto pre_o = [&]() -> bool {
    if (!spin_until(cx, cx.ctr_att, st.k1 * (uint32_t)SH::NKV, 10)) return false;
    const float* o = wsp<float>(a, a.off.o);
    for (int i = threadIdx.x; i < SH::ODIM; i += BLOCK) L.act[i] = ld_f32(o + i);
    __syncthreads();
    return true;
  };
  if (!mv<SH::FP8, SH::ODIM>(st.Ly->wo, 0, 0, r0, r1, L.act, L.outb, OUT_STORE, 1.f, pre_o)) return false;
  __syncthreads();
  float* h2 = wsp<float>(a, a.off.h2);
  for (int r = r0 + threadIdx.x; r < r1; r += BLOCK) st_f32(h2 + r, st.xs(r) + L.outb[r - r0]);
  arrive(cx, S_H2, st.k1, cx.nwg);
  return true;
}

// ------------------------------------------------------------------ stage: FFN gate/up (+ router)
// m[slot][j] = silu(gate_j . b) * (up_j . b) for rows [j0, j1) of one expert
template <class SH, typename Pre>
__device__ __forceinline__ bool gate_up(const KArgs& a, const Step& st, Lds& L, int expert, int slot, int j0, int j1,
                                        Pre&& pre) {
  const DLayer Ly = *gp(st.Ly);
  const size_t bo = (size_t)expert * Ly.gu_slot_bytes, so = (size_t)expert * Ly.gu_slot_scales;
  if (!mv<SH::FP8, SH::H>(Ly.w_gate, bo, so, j0, j1, L.act, L.outb, OUT_STORE, 1.f, pre)) return false;
  if (!mv<SH::FP8, SH::H>(Ly.w_up, bo, so, j0, j1, L.act, L.outc, OUT_STORE, 1.f, NoPre{})) return false;
  __syncthreads();
  float* mbuf = wsp<float>(a, a.off.m);
  for (int j = j0 + threadIdx.x; j < j1; j += BLOCK)
    st_f32(mbuf + (size_t)slot * SH::INTER + j, silu_f(L.outb[j - j0]) * L.outc[j - j0]);
  __syncthreads();
  return true;
}

template <class SH>
__device__ __forceinline__ bool stage_ffn(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  const int w = cx.w, nwg = cx.nwg;
  bool pending = true;
  // wait for h2, RMSNorm it into LDS; router workgroups compute their logit (fp64)
  auto pre_b = [&]() -> bool {
    if (!pending) return true;
    pending = false;
    if (!wait_all(cx, S_H2, st.k1, nwg)) return false;
    const float* h2 = wsp<float>(a, a.off.h2);
    rmsnorm_to_lds([&](int i) { return ld_f32(h2 + i); }, Ly.ffn_norm, SH::H, c.eps, L.act, L.red);
    if (w == 0)
      for (int i = threadIdx.x; i < SH::H; i += BLOCK) st_f32(wsp<float>(a, a.off.b_dbg) + i, L.act[i]);
    if constexpr (SH::MOE) {
      if (w < c.E) {
        const uint16_t* rrow = Ly.router + (size_t)w * SH::H;
        double s = 0.0;
        for (int q = threadIdx.x; q < SH::H / 8; q += BLOCK) s += dot8_bf16_f64(ld_g16(rrow + q * 8), L.act + q * 8);
        s = block_sum(s, L.red);
        if (threadIdx.x == 0) st_f64(wsp<double>(a, a.off.logits) + w, s);
      }
      arrive(cx, S_RT, st.k1, c.E);
    }
    return true;
  };
  const int j0 = split_at(SH::INTER, nwg, w), j1 = split_at(SH::INTER, nwg, w + 1);
  if constexpr (!SH::MOE) {
    if (!gate_up<SH>(a, st, L, 0, 0, j0, j1, pre_b)) return false;
  } else {
    // shared experts first: they do not depend on the router
    for (int sj = 0; sj < c.nshared; sj++)
      if (!gate_up<SH>(a, st, L, c.E + sj, c.topk + sj, j0, j1, pre_b)) return false;
    if (!pre_b()) return false;
    // router top-k (every workgroup computes the same selection)
    if (!wait_all(cx, S_RT, st.k1, c.E)) return false;
    double* lg = reinterpret_cast<double*>(L.outc);   // E doubles (outc is free here)
    const double* logits = wsp<double>(a, a.off.logits);
    for (int x = threadIdx.x; x < c.E; x += BLOCK) {
      const double r = ld_f64(logits + x);
      lg[x] = (c.router == PLD_ROUTER_SIGMOID_BIAS) ? (1.0 / (1.0 + exp(-r))) + (double)gp(Ly.router_bias)[x] : r;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      wave_topk(lg, c.E, c.topk, L.isel);
      if (threadIdx.x == 0) {
        double gsum = 0.0, tmp[32];
        if (c.router == PLD_ROUTER_SIGMOID_BIAS) {
          for (int s = 0; s < c.topk; s++) {
            tmp[s] = 1.0 / (1.0 + exp(-ld_f64(logits + L.isel[s])));
            gsum += tmp[s];
          }
        } else {
          const double mx = ld_f64(logits + L.isel[0]);
          for (int s = 0; s < c.topk; s++) {
            tmp[s] = exp(ld_f64(logits + L.isel[s]) - mx);
            gsum += tmp[s];
          }
        }
        for (int s = 0; s < c.topk; s++) L.fgate[s] = (float)(tmp[s] / gsum);
      }
    }
    __syncthreads();
    if (w == 0 && threadIdx.x < c.topk) {
      st_u32(reinterpret_cast<uint32_t*>(wsp<int>(a, a.off.sel)) + threadIdx.x, (uint32_t)L.isel[threadIdx.x]);
      st_f32(wsp<float>(a, a.off.gates) + threadIdx.x, L.fgate[threadIdx.x]);
    }
    // routed experts: this workgroup's share of the topk*inter (slot, row) pairs
    const int tot = c.topk * SH::INTER;
    const int i0 = split_at(tot, nwg, w), i1 = split_at(tot, nwg, w + 1);
    for (int s = i0 / SH::INTER; s < c.topk && s * SH::INTER < i1; s++) {
      const int lo = max(i0, s * SH::INTER) - s * SH::INTER, hi = min(i1, (s + 1) * SH::INTER) - s * SH::INTER;
      if (lo < hi && !gate_up<SH>(a, st, L, L.isel[s], s, lo, hi, NoPre{})) return false;
    }
  }
  arrive(cx, S_M, st.k1, nwg);
  return true;
}

// ------------------------------------------------------------------ stage: down projections + residual
template <class SH>
__device__ __forceinline__ bool stage_down(Ctx& cx, const KArgs& a, const Step& st, Lds& L, uint16_t* out_hidden) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  const int r0 = split_at(SH::H, cx.nwg, cx.w), r1 = split_at(SH::H, cx.nwg, cx.w + 1);
  bool pending = true;
  auto pre_m = [&]() -> bool {
    if (!pending) return true;
    pending = false;
    if (!wait_all(cx, S_M, st.k1, cx.nwg)) return false;
    const float* mbuf = wsp<float>(a, a.off.m);
    for (int i = threadIdx.x; i < c.slots * SH::INTER; i += BLOCK) L.act[i] = ld_f32(mbuf + i);
    for (int r = threadIdx.x; r < r1 - r0; r += BLOCK) L.outb[r] = 0.f;
    __syncthreads();
    return true;
  };
  for (int s = 0; s < c.slots; s++) {
    const int expert = !SH::MOE ? 0 : (s < c.topk ? L.isel[s] : c.E + (s - c.topk));
    const float gate = (!SH::MOE || s >= c.topk) ? 1.0f : L.fgate[s];
    const size_t bo = (size_t)expert * Ly.dn_slot_bytes, so = (size_t)expert * Ly.dn_slot_scales;
    if (!mv<SH::FP8, SH::INTER>(Ly.w_down, bo, so, r0, r1, L.act + (size_t)s * SH::INTER, L.outb, OUT_ACCUM, gate, pre_m))
      return false;
  }
  if (!pre_m()) return false;
  __syncthreads();
  const float* h2 = wsp<float>(a, a.off.h2);
  uint32_t* xb = wsp<uint32_t>(a, a.off.xbuf);
  for (int r = r0 + threadIdx.x; r < r1; r += BLOCK) {
    const uint32_t bits = f32_to_bf16(ld_f32(h2 + r) + L.outb[r - r0]);
    st_u32(xb + r, bits);
    if (out_hidden) gp(out_hidden)[r] = (uint16_t)bits;
  }
  arrive(cx, S_OUT, st.k1, cx.nwg);
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
      st.k1 = a.step0 + (uint32_t)(t * a.n_layers + li) + 1u;
      st.first = (t == 0 && li == 0);
      st.pos = a.pos0 + t;
      st.xs.p16 = st.first ? a.in_hidden : nullptr;
      st.xs.p32 = st.first ? nullptr : wsp<uint32_t>(a, a.off.xbuf);
      const bool last = (t == a.n_tokens - 1) && (li == a.n_layers - 1);
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
using ShapeTinyDense = GqaShape<256, 4, 4, 64, 1024, false, false>;
using ShapeGqaMoe = GqaShape<4096, 32, 8, 128, 1536, false, true>;

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
    int act = std::max({c->hidden, c->n_heads * c->head_dim, k->slots * c->inter, 2 * c->n_experts,
                        k->G * k->chmax + NWAVES * k->G * c->head_dim + 2 * k->G, 2 * k->G * k->cpg});
    k->act_floats = (int)al(act, 64);
    int outb = std::max({R / nwg + 4, c->hidden / nwg + 2, (k->slots * c->inter) / nwg + 2, c->inter / nwg + 2,
                         2 * c->n_experts + 2});
    k->outb_floats = (int)al(outb, 64);
    if (lds_bytes_for(k->act_floats, k->outb_floats) > 160 * 1024) return PLD_E_UNSUPPORTED;
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
  o.logits = p; p += al((size_t)std::max(k.E, 1) * 8);
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
  h->lds_bytes = lds_bytes_for(k.act_floats, k.outb_floats);
  h->steps = 0;
  h->bad = false;
  h->device = dev;
  h->last_stream = nullptr;
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
      {"logits", h->off.logits, (size_t)k.E * 8},
      {"sel", h->off.sel, (size_t)k.topk * 4},
      {"gates", h->off.gates, (size_t)k.topk * 4},
      {"m", h->off.m, (size_t)k.slots * k.inter * 4},
      {"x", h->off.xbuf, (size_t)k.H * 4},
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

pld_status pld_set_watchdog_us(pld_handle* h, int64_t us) {
  if (!h || us <= 0) return PLD_E_INVALID;
  h->budget = (long long)((double)us * h->wallclock_khz / 1000.0);
  if (h->budget < 1) h->budget = 1;
  return PLD_OK;
}

}  // extern "C"
