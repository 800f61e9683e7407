// KDA linear-attention decode stages of the persistent kernel (included by pld_kernel.hip
// after the shared stages; uses its Ctx / KArgs / Step / Lds, the LL handoff and the GEMV
// stream).
//
// KDA is the linear attention of the Kimi K3 article (section "FlashKDA Algorithm"): per
// head an fp32 state S [key channel][value channel] advanced once per token by the delta
// rule with a diagonal decay,
//   S' = diag(alpha) S,   u = beta (v - S'^T k),   S = S' + k u^T,   o = S^T q,
// with q, k, v from linear projections and a short causal convolution, q and k
// L2-normalised, alpha from a low-rank projection (the cumulative decay is written with
// exp2 on the page, so alpha = 2^g with g = -softplus(W_aup W_adown a)), beta = sigmoid of a
// down projection, and the head outputs normalised per head and gated by a linear output
// gate before the output projection (the paragraph after the algorithm, "Kimi Linear").
// The page's decode cost per head and token is ~7 D^2 FLOPs and 8 D^2 bytes (the state
// read and written), so the state step is bandwidth-bound like the weight GEMVs.
//
// One step of a KDA layer:
//   KX  a = RMSNorm(x); rows of [W_q; W_k; W_v; W_g; W_adown; W_beta] over all workgroups;
//       the q/k/v rows go through the width-4 causal convolution right where they are
//       produced (the ring of the three previous projection outputs lives in the caller's
//       cache, one fp32 per channel and position mod 3; a channel is always produced by the
//       same thread, so each ring entry is read and written by one thread)      -> LL kx
//   KS  workgroup (head h, 16 value columns): decay from W_aup (the head's 128 rows, kept
//       by each of its 8 workgroups), q/k norms, then the state step on its 128 x 16 block
//       of S (coherent loads and stores: the block is written by this thread one step
//       earlier)                                                                -> LL o
//   KO  per-head RMSNorm (gain o_norm) x output gate, then W_o + residual      -> LL h2
// then the shared FFN and down stages.
#pragma once

template <int H_, int NH_, int D_, int R_, int CW_, int INTER_, bool FP8_, bool MOE_>
struct KdaShape {
  static constexpr int H = H_, NH = NH_, D = D_, R = R_, CW = CW_, INTER = INTER_;
  static constexpr bool FP8 = FP8_, MOE = MOE_;
  static constexpr bool LUTX = false;
  static constexpr int QD = NH * D, ODIM = QD;
  static constexpr int NCH = 3 * QD;                 // convolution channels (q, k, v)
  static constexpr int ROWS = 4 * QD + R + NH;       // [W_q; W_k; W_v; W_g; W_adown; W_beta]
  static constexpr int CPW = 16;                      // value columns per state workgroup
  // LL block kx: [conv outputs 3 QD | gate QD | a_down R | beta NH]
  static constexpr int KX_GATE = NCH, KX_ALOW = 4 * QD, KX_BETA = 4 * QD + R, KX_WORDS = ROWS;
  static_assert(CW == 4 && D == 128 && R == 128 && FP8, "the compiled KDA layout");
};

// ------------------------------------------------------------------ KX: RMSNorm + projections + convolution
template <class SH>
__device__ __forceinline__ bool stage_x_kda(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const DLayer Ly = *gp(st.Ly);
  const int w = cx.w, nwg = cx.nwg;
  constexpr int R = SH::ROWS, QD = SH::QD, NCH = SH::NCH;
  constexpr size_t RB = (size_t)SH::H * (SH::FP8 ? 1 : 2);
  const int r0 = split_at(R, nwg, w), r1 = split_at(R, nwg, w + 1);   // host: r1 - r0 <= BLOCK
  int h0, h1;
  hrows(SH::H, nwg, w, &h0, &h1);
  RegVec<SH::H> gam;
  gam.load(Ly.attn_norm);
  // this thread's channel r0 + tid: its taps and the ring entries of the three previous
  // positions, loaded before the weight stream (after it they would queue behind it)
  const int pos = st.pos;
  const int rr = r0 + tid_opaque();
  const bool conv_row = rr < r1 && rr < NCH;
  float4 tp = make_float4(0.f, 0.f, 0.f, 0.f);
  float p1 = 0.f, p2 = 0.f, p3 = 0.f;   // projection outputs of positions pos-1, pos-2, pos-3
  if (conv_row) {
    tp = *reinterpret_cast<const PLD_GLOBAL float4*>(gp(Ly.conv_taps) + (size_t)rr * 4);
    p1 = ld_f32(Ly.conv_ring + (size_t)((pos + 2) % 3) * NCH + rr);
    p2 = ld_f32(Ly.conv_ring + (size_t)((pos + 1) % 3) * NCH + rr);
    p3 = ld_f32(Ly.conv_ring + (size_t)(pos % 3) * NCH + rr);
  }
  bool pending = true;
  auto pre_x = [&]() -> bool {
    if (!pending) return true;
    pending = false;
    return layer_input<SH::H, SH::FP8>(cx, a, st, L, gam, h0, h1);
  };
  {
    const DMat* mats[6] = {&Ly.wq, &Ly.wk, &Ly.wv, &Ly.w_g, &Ly.w_adown, &Ly.w_beta};
    constexpr int b[7] = {0, QD, 2 * QD, 3 * QD, 4 * QD, 4 * QD + SH::R, R};
    seg_begin();
    int ns = 0;
#pragma unroll
    for (int m = 0; m < 6; m++) {
      const int lo = max(r0, b[m]), hi = min(r1, b[m + 1]);
      if (lo < hi) {
        seg_set(L, ns, mats[m]->w + (size_t)(lo - b[m]) * RB, mats[m]->s, hi - lo, lo - b[m], 0, 1.f);
        ns++;
      }
    }
    seg_end();
    if (!gemv_list<SH::FP8, SH::H, PLD_IF_QKV>(L.segs, ns, L.act, L.outb, OUT_STORE, pre_x)) return false;
  }
  stamp(a, cx, st, TR_QKV_GEMV);
  if (!pre_x()) return false;
  __syncthreads();
  uint64_t* kx = wsp<uint64_t>(a, a.off.kx);
  const int r = rr;   // one row per thread (r1 - r0 <= BLOCK)
  if (r < r1) {
    const float v = L.outb[r - r0];
    if (r < NCH) {
      // causal convolution: the last tap on the current position
      const float y = fmaf(tp.x, p3, fmaf(tp.y, p2, fmaf(tp.z, p1, tp.w * v)));
      st_f32(Ly.conv_ring + (size_t)(pos % 3) * NCH + r, v);   // replaces the entry of pos - 3
      ll_put_f32(kx + r, y, st.k1);
    } else if (r < SH::KX_ALOW) {
      ll_put_f32(kx + r, 1.0f / (1.0f + __expf(-v)), st.k1);   // output gate
    } else if (r < SH::KX_BETA) {
      ll_put_f32(kx + r, v, st.k1);                             // decay projection (low rank)
    } else {
      ll_put_f32(kx + r, 1.0f / (1.0f + __expf(-v)), st.k1);   // beta
    }
  }
  stamp(a, cx, st, TR_QKV_DONE);
  return true;
}

// Sum over the lanes of a wave that share (lane & 3), result in every such lane.
__device__ __forceinline__ float sum_lanes_mod4(float v) {
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 8, 64);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// ------------------------------------------------------------------ KS: the state step of one (head, column block)
template <class SH>
__device__ __forceinline__ bool stage_state_kda(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  constexpr int D = SH::D, QD = SH::QD, R = SH::R, CPW = SH::CPW;
  constexpr int WPH = D / CPW;                       // workgroups per head (host: nwg == NH * WPH)
  const int h = cx.w / WPH, j0 = (cx.w % WPH) * CPW;
  const int tid = tid_opaque();
  const int lane = tid & 63, wave = tid >> 6;
  const int i = tid >> 2, jq = tid & 3;              // state row (key channel) and 4-column quarter
  // static weights first: row h*D + i of W_aup (R = 128 FP8 = 8 chunks; this thread's two)
  const size_t arow = (size_t)h * D + i;
  const uint4 wa0 = ld_stream16(Ly.w_aup.w + arow * R + jq * 32);
  const uint4 wa1 = ld_stream16(Ly.w_aup.w + arow * R + jq * 32 + 16);
  const float wsc = gp(Ly.w_aup.s)[arow >> 7];       // one 128-column block (R = 128)
  // this thread's 4 state entries S[h][i][j0 + 4 jq .. +4] (written by this thread one step earlier)
  float* sp = Ly.kstate + ((size_t)h * D + i) * D + j0 + 4 * jq;
  const uint4 sraw = ld_coh16(sp);
  // q, k of the head, v of the block, a_down, beta: one LL fetch
  float* qk = L.act;                 // [2 D]
  float* vv = qk + 2 * D;            // [CPW]
  float* al = vv + CPW;              // [R]
  float* bt = al + R;                // [1]
  float* wred = bt + 4;              // [NWAVES][CPW] wave partials
  float* uu = wred + NWAVES * CPW;   // [CPW]
  double* nrm = reinterpret_cast<double*>(uu + CPW + 4);   // [NWAVES]
  struct IdxKs {
    int h, j0;
    __device__ __forceinline__ int operator()(int n) const {
      if (n < D) return h * D + n;                                   // q
      if (n < 2 * D) return QD + h * D + (n - D);                    // k
      if (n < 2 * D + CPW) return 2 * QD + h * D + j0 + (n - 2 * D);  // v
      if (n < 2 * D + CPW + R) return SH::KX_ALOW + (n - 2 * D - CPW);
      return SH::KX_BETA + h;
    }
  };
  if (!ll_fetch<1>(cx, reinterpret_cast<uint32_t*>(qk), wsp<uint64_t>(a, a.off.kx), 2 * D + CPW + R + 1, st.k1, W_QKV,
                   IdxKs{h, j0}))
    return false;
  stamp(a, cx, st, TR_ATT_READY);
  // decay of key channel i: g = -softplus(W_aup[row] . a_down), alpha = 2^g (4 lanes per row)
  float z = 0.f;
  {
    float at[16];
#pragma unroll
    for (int e = 0; e < 16; e++) at[e] = al[jq * 32 + e];
    z = dot16_fp8(wa0, at);
#pragma unroll
    for (int e = 0; e < 16; e++) at[e] = al[jq * 32 + 16 + e];
    z += dot16_fp8(wa1, at);
    z *= wsc;
    z += __shfl_xor(z, 1, 64);
    z += __shfl_xor(z, 2, 64);
  }
  const float sp_z = fmaxf(z, 0.f) + log1pf(__expf(-fabsf(z)));
  const float alpha = exp2f(-sp_z);
  // q and k norms (fp64 sums): waves 0-1 square q, waves 2-3 square k
  {
    double sq = 0.0;
    if (tid < 2 * D) sq = (double)qk[tid] * (double)qk[tid];
    sq = wave_sum_any(sq);
    if (lane == 0) nrm[wave] = sq;
    __syncthreads();
  }
  const double qss = nrm[0] + nrm[1], kss = nrm[2] + nrm[3];
  const float qi = (float)((double)qk[i] / sqrt(qss + c.eps) / sqrt((double)D));
  const float ki = (float)((double)qk[D + i] / sqrt(kss + c.eps));
  const float beta = bt[0];
  float s4[4] = {__uint_as_float(sraw.x), __uint_as_float(sraw.y), __uint_as_float(sraw.z), __uint_as_float(sraw.w)};
#pragma unroll
  for (int e = 0; e < 4; e++) s4[e] *= alpha;              // S' = diag(alpha) S
  // column sums over the 128 rows: lanes with the same (lane & 3) in a wave, then the waves in order
  auto colsum = [&](const float* p4, float* out16) {
    float t[4];
#pragma unroll
    for (int e = 0; e < 4; e++) t[e] = sum_lanes_mod4(p4[e]);
    if (lane < 4)
#pragma unroll
      for (int e = 0; e < 4; e++) wred[wave * CPW + 4 * lane + e] = t[e];
    __syncthreads();
    if (tid < CPW) {
      float s = 0.f;
      for (int wv = 0; wv < NWAVES; wv++) s += wred[wv * CPW + tid];
      out16[tid] = s;
    }
    __syncthreads();
  };
  {
    float p4[4];
#pragma unroll
    for (int e = 0; e < 4; e++) p4[e] = s4[e] * ki;
    colsum(p4, uu);                                        // uu = S'^T k (this block's columns)
  }
  if (tid < CPW) uu[tid] = beta * (vv[tid] - uu[tid]);     // u = beta (v - S'^T k)
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 4; e++) s4[e] = fmaf(ki, uu[4 * jq + e], s4[e]);   // S = S' + k u^T
  // the new state block (coherent stores: read back by this thread at the next step)
  st_u64(reinterpret_cast<uint64_t*>(sp), ((uint64_t)__float_as_uint(s4[1]) << 32) | __float_as_uint(s4[0]));
  st_u64(reinterpret_cast<uint64_t*>(sp) + 1, ((uint64_t)__float_as_uint(s4[3]) << 32) | __float_as_uint(s4[2]));
  {
    float p4[4];
#pragma unroll
    for (int e = 0; e < 4; e++) p4[e] = s4[e] * qi;
    colsum(p4, uu);                                        // o = S^T q
  }
  uint64_t* ol = wsp<uint64_t>(a, a.off.o) + (size_t)h * D + j0;
  if (tid < CPW) ll_put_f32(ol + tid, uu[tid], st.k1);
  stamp(a, cx, st, TR_ATT_DONE);
  return true;
}

// ------------------------------------------------------------------ KO: head norm x gate, W_o + residual
template <class SH>
__device__ __forceinline__ bool stage_wo_kda(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  constexpr int QD = SH::QD, D = SH::D;
  static_assert(QD == 8 * BLOCK && D % 8 == 0, "8 elements of one head per thread");
  int r0, r1;
  hrows(SH::H, cx.nwg, cx.w, &r0, &r1);
  const int tid = tid_opaque();
  // this thread's 8 output-norm gains (elements 8 tid .. 8 tid + 7 lie in head tid / 16)
  const PLD_GLOBAL float4* gsrc = reinterpret_cast<const PLD_GLOBAL float4*>(gp(Ly.o_norm) + (8 * tid) % D);
  const float4 g0 = gsrc[0], g1 = gsrc[1];
  float* raw = L.act + apad<SH::FP8>(QD);   // [QD] o, then [QD] gate
  auto pre_o = [&]() -> bool {
    if (!ll_fetch<per_for(QD)>(cx, reinterpret_cast<uint32_t*>(raw), wsp<uint64_t>(a, a.off.o), QD, st.k1, W_O))
      return false;
    if (!ll_fetch<per_for(QD)>(cx, reinterpret_cast<uint32_t*>(raw + QD), wsp<uint64_t>(a, a.off.kx) + SH::KX_GATE, QD,
                               st.k1, W_QKV))
      return false;
    stamp(a, cx, st, TR_O_READY);
    float o8[8];
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      o8[e] = raw[8 * tid + e];
      ss += (double)o8[e] * (double)o8[e];
    }
    ss = dpp_sum_f64<16>(ss);   // the 16 threads of one head are one DPP row: valid in every lane of it
    const double rn = 1.0 / sqrt(ss / (double)D + c.eps);
    const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int e = 0; e < 8; e++)
      L.act[apad<SH::FP8>(8 * tid + e)] = (float)(((double)o8[e] * rn) * (double)gg[e]) * raw[QD + 8 * tid + e];
    __syncthreads();
    return true;
  };
  {
    const DMat wo = Ly.wo;
    seg_begin();
    seg_set(L, 0, wo.w + (size_t)r0 * QD * (SH::FP8 ? 1 : 2), wo.s, r1 - r0, r0, 0, 1.f);
    seg_end();
    if (!gemv_list<SH::FP8, QD, PLD_IF_WO>(L.segs, r1 > r0 ? 1 : 0, L.act, L.outb, OUT_STORE, pre_o)) return false;
  }
  __syncthreads();
  uint64_t* h2ll = wsp<uint64_t>(a, a.off.h2);
  for (int r = r0 + tid; r < r1; r += BLOCK) {
    const float v = L.xres[r - r0] + L.outb[r - r0];
    L.h2res[r - r0] = v;
    ll_put_f32(h2ll + r, v, st.k1);
  }
  stamp(a, cx, st, TR_WO_DONE);
  return true;
}

template <class SH>
__global__ void __launch_bounds__(BLOCK, 1) k_decode_kda(KArgs a) {
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
  int token = a.in_token;
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
      KArgs as = a;
      asm volatile("" : "+s"(as.ws));
      Ctx cs = cx;
      asm volatile("" : "+s"(cs.w), "+s"(cs.nwg));
      uint32_t lds0 = 0;
      asm volatile("" : "+s"(lds0));
      Lds L = carve(lds_raw + lds0, a.c);
      st.tr = L.tr;
      cs.wacc = (a.trace && st.idx < a.trace_steps) ? L.tr + TR_WAIT : nullptr;
      stamp(as, cs, st, TR_START);
      PLD_TEST_DELAY(a, cs.w, st.idx, 0);
      if (!stage_x_kda<SH>(cs, as, st, L)) return;
      PLD_TEST_DELAY(a, cs.w, st.idx, 1);
      if (!stage_state_kda<SH>(cs, as, st, L)) return;
      if (!stage_wo_kda<SH>(cs, as, st, L)) return;
      PLD_TEST_DELAY(a, cs.w, st.idx, 2);
      if (!stage_ffn<SH>(cs, as, st, L)) return;
      PLD_TEST_DELAY(a, cs.w, st.idx, 3);
      if (!stage_down<SH>(cs, as, st, L, last ? as.out_hidden : nullptr)) return;
      if constexpr (SH::FP8) {
        if (a.head_on && li == a.n_layers - 1 && !stage_head<SH>(cs, as, st, L, t, &token)) return;
      }
      trace_flush(as, cs, st);
    }
  }
}
