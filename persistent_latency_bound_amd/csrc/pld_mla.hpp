// MLA decode stages of the persistent kernel (included by pld_kernel.hip after the shared
// stages; uses its Ctx / KArgs / Step / Lds, the LL handoff and the GEMV stream).
//
// One step of an MLA layer, absorbed form (the latent cache is read once per head group):
//   X   a = RMSNorm(x); [c_q' ; c_kv' | k_r'] = [W_DQ ; W_DKV] a                    -> LL cqr, ckvr
//   Q   c_q = RMSNorm(c_q'); [q_nope | q_rope]_h = (W_UQ c_q)_h, RoPE on q_rope       -> LL qn, qr
//   ABS q_lat_h = W_UK_h^T q_nope_h                                                    -> LL qlat
//   ATT per (8-head group, token chunk): s = (q_lat.c_kv + q_rope.k_r)/sqrt(nope+rope),
//       online softmax, o_lat partial = P.c_kv; MFMA 16x16x16 bf16 for both products -> LL part
//   MRG o_lat_h = merge of the chunk partials                                          -> LL olat
//   UV  o_h = W_UV_h o_lat_h                                                           -> LL o
// then the shared output projection, FFN and down stages.
// The absorbed form is the one the Kimi Linear discussion of the Kimi K3 article relies on
// (attention over the compressed latent with the up-projections folded into q and o).
#pragma once

template <int H_, int NH_, int QL_, int KL_, int RD_, int ND_, int VD_, int INTER_, bool FP8_, bool MOE_, bool SPARSE_,
          int IH_ = 0, int ID_ = 0, int HPW_ = 8, bool LUTX_ = false>
struct MlaShape {
  static constexpr int H = H_, NH = NH_, QL = QL_, KL = KL_, RD = RD_, ND = ND_, VD = VD_, INTER = INTER_;
  static constexpr bool FP8 = FP8_, MOE = MOE_, SPARSE = SPARSE_;
  static constexpr bool LUTX = LUTX_;   // expert matrices as LUT3 (3-bit indices, 8-entry E4M3 codebooks)
  static_assert(!LUTX || FP8, "LUT3 experts sit in an FP8 layer (padded activation layout)");
  static constexpr int IH = IH_, ID = ID_;        // indexer heads and key width (sparse layers)
  static_assert(!SPARSE || (!FP8 && IH > 0 && ID > 0), "the sparse layer has bf16 weights and an indexer");
  static constexpr int LAT = KL + RD, QH = ND + RD, ODIM = NH * VD;
  static constexpr int HPW = HPW_, NHG = NH / HPW;   // heads per attention workgroup (8 or 16), head groups
  static_assert(HPW == 8 || HPW == 16, "one or two heads per wave");
  static constexpr int TB = 32;                   // latent rows per attention sub-block
  static constexpr int CSTR = LAT + 4;            // LDS row stride (bf16) of a staged latent row
  static_assert(NH % HPW == 0 && LAT % 64 == 0 && KL % 16 == 0 && RD % 2 == 0 && ND % 2 == 0, "MLA shape");
};

typedef short bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ short bf16_bits(float f) { return (short)f32_to_bf16(f); }

// Coherent 16-byte read of a latent row written inside this launch.
__device__ __forceinline__ uint4 ld_coh16(const void* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t x = ld_u64(q), y = ld_u64(q + 1);
  return make_uint4((uint32_t)x, (uint32_t)(x >> 32), (uint32_t)y, (uint32_t)(y >> 32));
}

// ------------------------------------------------------------------ X: RMSNorm + [W_DQ ; W_DKV (; W_w ; W_kI)]
// The sparse layer accumulates these rows in fp64: c_q' feeds the indexer's selection,
// an integer result, so it travels as fp64 (two LL words per value) and the indexer head
// weights w and key k_I are rounded to fp32 once, from fp64 sums.
// Attention partial of one (head, chunk) (and position, in the batched path): LL words
// [m, l, 14 spare | acc as fp16 pairs]; the acc words start one 128-byte line after the row
// start and rows are whole lines, so stores that cover 16 consecutive words write whole lines
// (8-byte stores of half a line each from every workgroup at once were twice as many partial
// line writes).
constexpr int VP_ACC = 16;
template <int KL>
__host__ __device__ constexpr int vp_stride() { return KL / 2 + VP_ACC; }

template <class SH>
__device__ __forceinline__ bool stage_x_mla(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const DLayer Ly = *gp(st.Ly);
  const int w = cx.w, nwg = cx.nwg;
  constexpr int NIX = SH::SPARSE ? SH::IH + SH::ID : 0;
  constexpr int R = SH::QL + SH::LAT + NIX;
  constexpr size_t RB = (size_t)SH::H * (SH::FP8 ? 1 : 2);
  const int r0 = split_at(R, nwg, w), r1 = split_at(R, nwg, w + 1);
  int h0, h1;
  hrows(SH::H, nwg, w, &h0, &h1);
  RegVec<SH::H> gam;
  gam.load(Ly.attn_norm);
  bool pending = true;
  auto pre_x = [&]() -> bool {
    if (!pending) return true;
    pending = false;
    return layer_input<SH::H, SH::FP8>(cx, a, st, L, gam, h0, h1);
  };
  {
    constexpr int NM = SH::SPARSE ? 4 : 2;
    const DMat* mats[4] = {&Ly.w_dq, &Ly.w_dkv, &Ly.w_w, &Ly.w_ki};
    constexpr int b[5] = {0, SH::QL, SH::QL + SH::LAT, SH::QL + SH::LAT + SH::IH, R};
    seg_begin();
    int ns = 0;
#pragma unroll
    for (int m = 0; m < NM; m++) {
      const int lo = max(r0, b[m]), hi = min(r1, b[m + 1]);
      if (lo < hi) {
        seg_set(L, ns, mats[m]->w + (size_t)(lo - b[m]) * RB, mats[m]->s, hi - lo, lo - b[m], 0, 1.f);
        ns++;
      }
    }
    seg_end();
    if (!gemv_list<SH::FP8, SH::H, PLD_IF_QKV, SH::SPARSE>(L.segs, ns, L.act, L.outb, OUT_STORE, pre_x)) return false;
  }
  stamp(a, cx, st, TR_QKV_GEMV);
  if (!pre_x()) return false;
  __syncthreads();
  uint64_t* cqr = wsp<uint64_t>(a, a.off.cqr);
  uint64_t* ckvr = wsp<uint64_t>(a, a.off.ckvr);
  for (int r = r0 + tid_opaque(); r < r1; r += BLOCK) {
    if constexpr (SH::SPARSE) {
      const double v = reinterpret_cast<const double*>(L.outb)[r - r0];
      if (r < SH::QL) {
        const uint64_t bits = (uint64_t)__double_as_longlong(v);
        ll_put(cqr + 2 * r, (uint32_t)bits, st.k1);
        ll_put(cqr + 2 * r + 1, (uint32_t)(bits >> 32), st.k1);
      } else if (r < SH::QL + SH::LAT) {
        ll_put_f32(ckvr + (r - SH::QL), (float)v, st.k1);
      } else {
        ll_put_f32(wsp<uint64_t>(a, a.off.ixr) + (r - SH::QL - SH::LAT), (float)v, st.k1);
      }
    } else {
      const float v = L.outb[r - r0];
      if (r < SH::QL) ll_put_f32(cqr + r, v, st.k1);
      else ll_put_f32(ckvr + (r - SH::QL), v, st.k1);
    }
  }
  stamp(a, cx, st, TR_QKV_DONE);
  return true;
}

// RMSNorm of an fp64 vector held as (lo, hi) 32-bit word pairs in LDS, written as fp32 into
// the activation layout apad<PAD>: dst[apad<PAD>(i)] = fp32((x_i * r) * gamma_i),
// r = 1/sqrt(sum(x^2)/N + eps), all in fp64.
template <int N, bool PAD>
__device__ __forceinline__ void rmsnorm_f64src(float* dst, const uint32_t* src, const RegVec<N>& gam, double eps,
                                               double* red) {
  auto x_at = [&](int i) -> double {
    return __longlong_as_double((long long)(((uint64_t)src[2 * i + 1] << 32) | src[2 * i]));
  };
  double xv[RegVec<N>::K];   // kept in registers between the passes (see rmsnorm_reg)
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < RegVec<N>::K; k++) {
    const int i = tid_opaque() + k * BLOCK;
    xv[k] = (N % BLOCK == 0 || i < N) ? x_at(i) : 0.0;
    ss += xv[k] * xv[k];
  }
  ss = block_sum(ss, red);
  const double r = 1.0 / sqrt(ss / (double)N + eps);
#pragma unroll
  for (int k = 0; k < RegVec<N>::K; k++) {
    const int i = tid_opaque() + k * BLOCK;
    if (N % BLOCK == 0 || i < N) dst[apad<PAD>(i)] = (float)((xv[k] * r) * (double)gam.v[k]);
  }
  __syncthreads();
}

// ------------------------------------------------------------------ Q: RMSNorm(c_q) + W_UQ (+ W_qI) + RoPE
// Sparse layer: c_q' arrives in fp64 and is normalised to fp32 exactly as the indexer's
// definition has it; the W_qI rows (indexer queries) accumulate in fp64 and are rounded
// to bf16 once, from the fp64 sum.
template <class SH>
__device__ __forceinline__ bool stage_q_mla(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  const int w = cx.w, nwg = cx.nwg;
  constexpr int RQ = SH::NH * SH::QH;
  constexpr int NQI = SH::SPARSE ? SH::IH * SH::ID : 0;
  constexpr int R = RQ + NQI;
  constexpr size_t RB = (size_t)SH::QL * (SH::FP8 ? 1 : 2);
  static_assert(RQ % 2 == 0 && NQI % 2 == 0, "row pairs");
  const int r0 = 2 * split_at(R / 2, nwg, w), r1 = 2 * split_at(R / 2, nwg, w + 1);
  RegVec<SH::QL> gq;
  gq.load(Ly.q_norm);
  bool pending = true;
  auto pre_q = [&]() -> bool {
    if (!pending) return true;
    pending = false;
    if constexpr (SH::SPARSE) {
      uint32_t* raw = reinterpret_cast<uint32_t*>(L.act + apad<SH::FP8>(SH::QL));   // [2*QL] fp64 words
      if (!ll_fetch<per_for(2 * SH::QL)>(cx, raw, wsp<uint64_t>(a, a.off.cqr), 2 * SH::QL, st.k1, W_CQ)) return false;
      rmsnorm_f64src<SH::QL, SH::FP8>(L.act, raw, gq, c.eps, L.red);
    } else {
      if (!ll_fetch<per_for(SH::QL)>(cx, reinterpret_cast<uint32_t*>(L.act), wsp<uint64_t>(a, a.off.cqr), SH::QL,
                                     st.k1, W_CQ, IdxLinear{}, StPad<SH::FP8>{}))
        return false;
      rmsnorm_reg<SH::QL, SH::FP8>(L.act, gq, c.eps, L.red);
    }
    stamp(a, cx, st, TR_CQ_READY);
    return true;
  };
  // RoPE (cos, sin) of this thread's first output pair, loaded before the GEMV: after it,
  // a global load would queue behind the GEMV's trailing weight loads
  const PLD_GLOBAL float* rope = gp(wsp<float>(a, a.off.rope)) + (size_t)st.pos * SH::RD;   // (cos, sin) pairs
  float rcs = 1.f, rsn = 0.f;
  {
    const int r = 2 * (r0 / 2 + tid_opaque()), k = r % SH::QH;
    if (r < r1 && r < RQ && k >= SH::ND) {
      rcs = rope[k - SH::ND];
      rsn = rope[k - SH::ND + 1];
    }
  }
  seg_begin();
  int ns = 0;
  if (r0 < RQ) {
    seg_set(L, ns, Ly.w_uq.w + (size_t)r0 * RB, Ly.w_uq.s, min(r1, RQ) - r0, r0, 0, 1.f);
    ns++;
  }
  if (r1 > RQ) {
    const int lo = max(r0, RQ) - RQ;
    seg_set(L, ns, Ly.w_qi.w + (size_t)lo * RB, Ly.w_qi.s, r1 - max(r0, RQ), lo, 0, 1.f);
    ns++;
  }
  seg_end();
  if (!gemv_list<SH::FP8, SH::QL, PLD_IF_WO, SH::SPARSE>(L.segs, ns, L.act, L.outb, OUT_STORE, pre_q)) return false;
  if (!pre_q()) return false;
  stamp(a, cx, st, TR_Q_GEMV);
  __syncthreads();
  auto outv = [&](int i) -> float {
    if constexpr (SH::SPARSE) return (float)reinterpret_cast<const double*>(L.outb)[i];
    else return L.outb[i];
  };
  uint64_t* qn = wsp<uint64_t>(a, a.off.q);
  uint64_t* qr = wsp<uint64_t>(a, a.off.qr);
  for (int p = r0 / 2 + tid_opaque(); p < r1 / 2; p += BLOCK) {
    const int r = 2 * p, h = r / SH::QH, k = r % SH::QH;
    if (SH::SPARSE && r >= RQ) {   // indexer query pair, bf16 from fp64
      const double* od = reinterpret_cast<const double*>(L.outb);
      ll_put(wsp<uint64_t>(a, a.off.qi) + (r - RQ) / 2,
             f64_to_bf16(od[r - r0]) | (f64_to_bf16(od[r + 1 - r0]) << 16), st.k1);
      continue;
    }
    const float v0 = outv(r - r0), v1 = outv(r + 1 - r0);
    if (k < SH::ND) {
      ll_put_f32(qn + h * SH::ND + k, v0, st.k1);
      ll_put_f32(qn + h * SH::ND + k + 1, v1, st.k1);
    } else {
      // q_rope as bf16 pairs: the attention's matrix cores take it in bf16 (same rounding)
      const int d = k - SH::ND;
      const bool first = p == r0 / 2 + tid_opaque();
      const float cs = first ? rcs : rope[d], sn = first ? rsn : rope[d + 1];
      ll_put(qr + (h * SH::RD + d) / 2, f32_to_bf16(v0 * cs - v1 * sn) | (f32_to_bf16(v0 * sn + v1 * cs) << 16),
             st.k1);
    }
  }
  stamp(a, cx, st, TR_ATT_Q);
  return true;
}

// ------------------------------------------------------------------ IDX: indexer scores of the T = pos + 1 tokens
// The sparse indexer of the TileRT article ("But What Exactly is TileRT?", its Sparse
// Indexer worker): every cached token t has an FP8 key row (E4M3 codes + fp32 scale s_t);
// its score is sum_h w_h * max(0, s_t * sum_i q_I[h,i] * dec(code_t,i)). The selection is
// an integer result decided by these scores, so they are computed exactly as defined: in
// fp64, i ascending, then h ascending, each product rounded on its own before its add.
// (q_I is bf16 and a decoded code has 4 significant bits, so q_I * dec is exact in fp64
// and a fused multiply-add of it rounds exactly once, like the separate add.)
// Workgroup w scores tokens t = w + i*nwg (interleaved, so that each workgroup's keys are
// a sample of the whole cache); four lanes per token, each with two heads. The workgroup
// holding the new token encodes its key (fp32 scale amax/448, fp32 quotient, E4M3 round to
// nearest even) and appends it to the cache. Scores leave as order-preserving 64-bit keys
// (two u32 halves, coherent stores, read only when the selection falls back to every
// token). Each workgroup then ranks its own keys and publishes its SEL_LIST largest as a
// list: the high halves as LL words in rank order, the low halves and token indices in
// plain memory written before them (0 marks an empty slot: no score's key is 0).
constexpr int SEL_LKMAX = 256;   // keys per scoring workgroup: T <= SEL_LKMAX * nwg
constexpr int SEL_LIST = 40;     // keys each scoring workgroup publishes, in rank order
template <class SH>
__device__ __forceinline__ bool stage_idx_mla(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  constexpr int IH = SH::IH, ID = SH::ID;
  static_assert(IH == 8 && ID == 64, "indexer lanes: 4 lanes x 2 heads per token, 64-byte key rows");
  constexpr int TPR = BLOCK / 4;   // tokens per round
  const DLayer Ly = *gp(st.Ly);
  const uint32_t k1 = st.k1;
  const int tid = tid_opaque();
  const int pos = st.pos, T = pos + 1, nwg = cx.nwg, w = cx.w;
  const int nt = w < T ? (T - 1 - w) / nwg + 1 : 0;   // this workgroup's tokens w + i*nwg, i < nt
  uint64_t* ilist = wsp<uint64_t>(a, a.off.ilist) + (size_t)w * SEL_LIST;
  if (nt == 0) {   // no tokens here: an empty list (the selector reads every workgroup's)
    if (tid < SEL_LIST) ll_put(ilist + tid, 0u, k1);
    return true;
  }
  const int fresh = a.pos0;   // rows >= fresh were written inside this launch
  const bool owner = pos % nwg == w;
  // LDS
  double* qd = reinterpret_cast<double*>(L.act);           // [ID][IH] q_I as fp64
  double* wd = qd + ID * IH;                                // [IH] head weights
  uint64_t* lk = reinterpret_cast<uint64_t*>(wd + IH);      // [SEL_LKMAX] this workgroup's keys
  uint32_t* raw = reinterpret_cast<uint32_t*>(lk + SEL_LKMAX);   // [IH*ID/2] q_I bf16 pairs, [IH] w, [ID] k_I
  uint32_t* ncw = raw + IH * ID / 2 + IH + ID;              // [ID/4] code words of the new row, [1] its scale
  uint32_t* lhi = ncw + ID / 4 + 2;                         // [SEL_LIST] high halves of the published list
  const int hp = tid & 3;
  // key rows of both rounds (a workgroup has at most 2 * TPR tokens), issued before the
  // wait for q_I so that neither round pays its own load latency afterwards
  uint4 cw[2][4];
  float ks[2];
  auto load_rows = [&](int rd) {
    const int tt = w + min(rd * TPR + (tid >> 2), nt - 1) * nwg;
    const uint8_t* row = Ly.icodes + (size_t)tt * ID;
    if (tt >= fresh) {
#pragma unroll
      for (int q = 0; q < 4; q++) cw[rd][q] = ld_coh16(row + 16 * q);
      ks[rd] = ld_f32(Ly.iscales + tt);
    } else {
#pragma unroll
      for (int q = 0; q < 4; q++) cw[rd][q] = ld_g16(row + 16 * q);
      ks[rd] = gp(Ly.iscales)[tt];
    }
  };
  load_rows(0);
  if (nt > TPR) load_rows(1);
  // q_I (Q stage), w and, for the new token's workgroup, k_I (X stage)
  {
    const uint32_t qiw = (uint32_t)(a.off.qi / 8), ixw = (uint32_t)(a.off.ixr / 8);
    auto idx = [=](int i) -> int { return i < IH * ID / 2 ? (int)qiw + i : (int)ixw + (i - IH * ID / 2); };
    const int nw = IH * ID / 2 + IH + (owner ? ID : 0);
    if (!ll_fetch<1>(cx, raw, reinterpret_cast<const uint64_t*>(a.ws), nw, k1, W_IX, idx)) return false;
  }
  for (int i = tid; i < IH * ID; i += BLOCK) {
    const int h = i / ID, k = i % ID;
    const uint32_t pr = raw[i / 2];
    qd[k * IH + h] = (double)((i & 1) ? bf_hi(pr) : bf_lo(pr));
  }
  if (tid < IH) wd[tid] = (double)__uint_as_float(raw[IH * ID / 2 + tid]);
  if (tid < SEL_LIST) lhi[tid] = 0u;   // entries past this workgroup's tokens stay padding (0)
  if (owner && tid < 64) {   // one wave: the new key row (ID == 64 lanes)
    const float k = __uint_as_float(raw[IH * ID / 2 + IH + tid]);
    const float amax = wave_max(fabsf(k));
    const float sig = amax > 0.f ? (float)((double)amax / 448.0) : 1.0f;
    const float quo = fminf(fmaxf((float)((double)k / (double)sig), -448.f), 448.f);
    reinterpret_cast<uint8_t*>(ncw)[tid] = (uint8_t)e4m3_encode(quo);
    if (tid == 0) reinterpret_cast<float*>(ncw)[ID / 4] = sig;
  }
  __syncthreads();
  if (owner && tid < ID / 4 + 1) {   // cache append (coherent stores; drained before the done word)
    if (tid < ID / 4) st_u32(reinterpret_cast<uint32_t*>(Ly.icodes + (size_t)pos * ID) + tid, ncw[tid]);
    else st_u32(reinterpret_cast<uint32_t*>(Ly.iscales + pos), ncw[ID / 4]);
  }
  uint32_t* kh = wsp<uint32_t>(a, a.off.ikh);
  uint32_t* kl = wsp<uint32_t>(a, a.off.ikl);
#pragma unroll
  for (int rd = 0; rd < 2; rd++) {
    if (rd * TPR >= nt) break;
    const int i = rd * TPR + (tid >> 2);
    const int tt = w + i * nwg;
    uint32_t wv[16] = {cw[rd][0].x, cw[rd][0].y, cw[rd][0].z, cw[rd][0].w, cw[rd][1].x, cw[rd][1].y,
                       cw[rd][1].z, cw[rd][1].w, cw[rd][2].x, cw[rd][2].y, cw[rd][2].z, cw[rd][2].w,
                       cw[rd][3].x, cw[rd][3].y, cw[rd][3].z, cw[rd][3].w};
    float sc = ks[rd];
    if (tt == pos) {
#pragma unroll
      for (int j = 0; j < 16; j++) wv[j] = ncw[j];
      sc = reinterpret_cast<const float*>(ncw)[ID / 4];
    }
    double d0 = 0.0, d1 = 0.0;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[j], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[j], true);
      const float dv[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const double2 q2 = *reinterpret_cast<const double2*>(qd + (4 * j + e) * IH + 2 * hp);
        d0 = fma(q2.x, (double)dv[e], d0);
        d1 = fma(q2.y, (double)dv[e], d1);
      }
    }
    double score;
    {
#pragma clang fp contract(off)
      const double s64 = (double)sc;
      const double r0 = fmax(s64 * d0, 0.0), r1 = fmax(s64 * d1, 0.0);
      const double p0 = wd[2 * hp] * r0, p1 = wd[2 * hp + 1] * r1;
      // the 8 products of the token, from the 4 lanes of its quad, added in head order
      const double p[8] = {dpp_mov_f64<0x00, 0xf, false>(p0), dpp_mov_f64<0x00, 0xf, false>(p1),
                           dpp_mov_f64<0x55, 0xf, false>(p0), dpp_mov_f64<0x55, 0xf, false>(p1),
                           dpp_mov_f64<0xAA, 0xf, false>(p0), dpp_mov_f64<0xAA, 0xf, false>(p1),
                           dpp_mov_f64<0xFF, 0xf, false>(p0), dpp_mov_f64<0xFF, 0xf, false>(p1)};
      score = 0.0;
#pragma unroll
      for (int h = 0; h < IH; h++) score = score + p[h];
    }
    if (score == 0.0) score = 0.0;   // one key for +0 and -0
    const uint64_t bits = (uint64_t)__double_as_longlong(score);
    const uint64_t key = (bits >> 63) ? ~bits : (bits | (1ull << 63));
    if (hp == 0 && i < nt) {
      st_u32(kh + tt, (uint32_t)(key >> 32));
      st_u32(kl + tt, (uint32_t)key);
      lk[i] = key;
    }
  }
  __syncthreads();
  {   // local ranks (key desc, token asc), four lanes per key; the top SEL_LIST form the list
    uint32_t* llo = wsp<uint32_t>(a, a.off.ilo) + (size_t)w * SEL_LIST;
    uint32_t* ltk = wsp<uint32_t>(a, a.off.itok) + (size_t)w * SEL_LIST;
    for (int c0 = 0; c0 < nt; c0 += TPR) {
      const int c = c0 + (tid >> 2);
      int rank = 0;
      uint64_t kc = 0;
      if (c < nt) {
        kc = lk[c];
#pragma unroll 8
        for (int d = hp; d < nt; d += 4) {
          const uint64_t kd = lk[d];
          rank += (kd > kc || (kd == kc && d < c)) ? 1 : 0;
        }
      }
      rank += __shfl_xor(rank, 1, 64);
      rank += __shfl_xor(rank, 2, 64);
      if (c < nt && hp == 0 && rank < SEL_LIST) {
        lhi[rank] = (uint32_t)(kc >> 32);
        st_u32(llo + rank, (uint32_t)kc);
        st_u32(ltk + rank, (uint32_t)(w + c * nwg));
      }
    }
  }
  vm_wait();   // key halves, list low halves and tokens (and a new key row) before the list words
  __syncthreads();
  if (tid < SEL_LIST) ll_put(ilist + tid, lhi[tid], k1);
  stamp(a, cx, st, TR_IDX_DONE);
  return true;
}

// ------------------------------------------------------------------ SEL: exact top-k of the indexer keys
// One workgroup selects the K = min(topk, T) largest keys (ties to the lower token index,
// the order the selection is defined with) and publishes the chosen token indices in
// ascending order as LL words.
//  * Bound: with r = ceil(K / nwg), every scorer holds r keys at or above its r-th largest,
//    so the K-th largest key of all is at least the smallest of those r-th keys (0 if a
//    scorer holds fewer than r). A scorer's unlisted keys are at most its last listed key;
//    when that key's high half is below the bound for every scorer, the lists hold every
//    key that can be chosen and the selection runs over the list entries alone (20 per
//    thread). Otherwise sel_all_tokens takes the same steps over every token.
//  * Radix select, most significant digit first (5-bit digits, starting below the bits
//    all candidates share): each pass adds every entry's candidacy into per-lane private
//    16-bit counters in LDS (lane-owned columns: no atomic contention, no bank conflicts,
//    no branches), sums the 32 bins and keeps the bin that holds the K-th key; entries in
//    higher bins are taken.
//  * Once at most SEL_CMAX candidates are left they are ranked directly by (key, index)
//    with the full 64-bit keys; if the high halves tie among more candidates than that,
//    the low halves get the same passes, and fully equal keys are cut by token index.
//  * Taken tokens are set in an LDS bitmap; the output walks it in contiguous per-thread
//    ranges with one block-wide exclusive scan, which gives ascending order.
constexpr int SEL_WG = 0;
constexpr int SEL_MAXJ = 68;                  // all-token path: token columns per thread, T <= SEL_MAXJ * BLOCK
constexpr int SEL_MAXWG = 256;                // scoring workgroups whose lists fit the LDS region
constexpr int SEL_LENT = SEL_MAXWG * SEL_LIST;   // list entries
constexpr int SEL_EPT = SEL_LENT / BLOCK;     // list entries per thread
constexpr int SEL_CMAX = 128;                 // candidates ranked directly
constexpr int SEL_ROWS = 16;                  // counter words per lane: 32 bins of 16 bits
constexpr int SEL_BMW = 3;                    // bitmap words per thread: tokens [96 tid, 96 tid + 96)
static_assert(SEL_LENT % BLOCK == 0 && SEL_BMW * 32 >= SEL_MAXJ && SEL_EPT % 4 == 0, "selector tiling");
// LDS words: counters | fetched lists | token bitmap | scalars | rank lists
constexpr int SEL_LDS_WORDS = SEL_ROWS * BLOCK + SEL_LENT + SEL_BMW * BLOCK + 64 + 3 * SEL_CMAX;
static_assert(SEL_MAXJ * BLOCK / 4 <= SEL_LENT, "all-token flags share the list region");

// Exclusive prefix sum of v over the workgroup (thread order); every thread must call.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum) {
  const int tid = tid_opaque(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t x = wave_incl_scan_u32(v);
  __syncthreads();
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t off = 0;
  for (int w = 0; w < wave; w++) off += wsum[w];
  return off + x - v;
}

struct SelLds {
  uint32_t *hist, *lst, *bm, *sv, *tot, *wsum, *chi, *clo, *ctk;
  uint8_t* fl;
};
__device__ __forceinline__ SelLds sel_carve(float* act) {
  SelLds S;
  S.hist = reinterpret_cast<uint32_t*>(act);     // [SEL_ROWS][BLOCK] packed 16-bit counters
  S.lst = S.hist + SEL_ROWS * BLOCK;              // [SEL_LENT] list entries: key high halves
  S.fl = reinterpret_cast<uint8_t*>(S.lst);      // [SEL_MAXJ*BLOCK] token flags (all-token path)
  S.bm = S.lst + SEL_LENT;                        // [SEL_BMW*BLOCK] taken tokens
  S.sv = S.bm + SEL_BMW * BLOCK;                  // [16] scalars
  S.tot = S.sv + 16;                              // [16] bin-pair totals
  S.wsum = S.tot + 16;                            // [32] scan / reduction partials
  S.chi = S.wsum + 32;                            // [SEL_CMAX] ranked candidates: key high half
  S.clo = S.chi + SEL_CMAX;                       //   low half
  S.ctk = S.clo + SEL_CMAX;                       //   token
  return S;
}

// The selected tokens, staged by rank in the counter words (free once the passes are
// done; at most SEL_ROWS * BLOCK of them), written out by every thread at once. Stores
// issued from the per-word bit loops instead each waited for the previous loop's stores
// to complete.
constexpr int SEL_STAGE_MAX = SEL_ROWS * BLOCK;
__device__ __forceinline__ void sel_write_out(const SelLds& S, uint64_t* isel, int K, uint32_t k1) {
  __syncthreads();
  for (int j = tid_opaque(); j < K; j += BLOCK) ll_put(isel + j, S.hist[j], k1);
}

// After a counting pass: bin totals (each thread clears the counters it read), the bin
// holding the need-th largest candidate; need and ncand updated. `pad` non-candidates were
// counted in bin 0.
__device__ __forceinline__ uint32_t sel_finish_pass(const SelLds& S, uint32_t nb, uint32_t pad, int& need, int& ncand) {
  const int tid = tid_opaque(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __syncthreads();
  {
    const int wr = tid >> 5, sg = tid & 31;   // 16 rows x 32 segments of 16 counters
    uint4* src = reinterpret_cast<uint4*>(S.hist + wr * BLOCK + sg * 16);
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const uint4 v = src[q];
      sum += v.x + v.y + v.z + v.w;
    }
    uint32_t z = 0u;   // made here, not a zero vector hoisted to kernel entry
    asm volatile("" : "+v"(z));
#pragma unroll
    for (int q = 0; q < 4; q++) src[q] = make_uint4(z, z, z, z);
    sum = row16_sum_u32(sum);
    sum += dpp_u32<0x142, 0xa, true>(sum);   // rows 0+1 (and 2+3): valid in lanes 16..31, 48..63
    if (sg == 31) S.tot[wr] = sum;
  }
  __syncthreads();
  if (wave == 0) {
    // lane L holds bin nb-1-L, so the inclusive scan over lanes counts the bins at or above
    // it; the first lane where that reaches need holds the bin of the need-th largest
    const int bn = (int)nb - 1 - lane;
    uint32_t c = 0u;
    if (bn >= 0) {
      const uint32_t tw = S.tot[bn >> 1];
      c = ((bn & 1) ? tw >> 16 : tw & 0xffffu) - (bn == 0 ? pad : 0u);
    }
    const uint32_t cum = wave_incl_scan_u32(c);
    const uint64_t m = __ballot(bn >= 0 && cum >= (uint32_t)need);
    const int L = __ffsll((unsigned long long)m) - 1;
    const uint32_t cb = (uint32_t)__builtin_amdgcn_readlane((int)c, L);
    const uint32_t cumb = (uint32_t)__builtin_amdgcn_readlane((int)cum, L);
    if (lane == 0) {
      S.sv[0] = nb - 1u - (uint32_t)L;
      S.sv[1] = (uint32_t)need - (cumb - cb);
      S.sv[2] = cb;
    }
  }
  __syncthreads();
  need = (int)S.sv[1];
  ncand = (int)S.sv[2];
  return S.sv[0];
}
// Counting of NC register columns: adds the candidacy of column j's digit (val(j) >> shift) & nbm1.
template <int NC, typename V, typename C>
__device__ __forceinline__ void sel_count(const SelLds& S, V&& val, C&& is_cand, int shift, uint32_t nbm1) {
  const int tid = tid_opaque();
#pragma unroll
  for (int j = 0; j < NC; j++) {
    const uint32_t d = (val(j) >> shift) & nbm1;
    const uint32_t inc = (uint32_t)is_cand(j) << ((d & 1u) << 4);
    __hip_atomic_fetch_add(lds_ptr(&S.hist[(d >> 1) * BLOCK + tid]), inc, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}
// 8-bit digit passes (the list path): each wave adds its candidates' digits
// (val(j) >> shift) & nbm1 into its own 256-bin histogram in LDS (S.hist rows, zero
// before the first pass; sel_finish8 clears what it reads).
template <int NC, typename V, typename C>
__device__ __forceinline__ void sel_count8(const SelLds& S, V&& val, C&& is_cand, int shift, uint32_t nbm1) {
  const int wave = __builtin_amdgcn_readfirstlane(tid_opaque() >> 6);
  uint32_t* hw = S.hist + wave * 256;
#pragma unroll
  for (int j = 0; j < NC; j++) {
    if (is_cand(j)) {
      const uint32_t d = (val(j) >> shift) & nbm1;
      __hip_atomic_fetch_add(lds_ptr(&hw[d]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
}
// After sel_count8 with nb <= 256 bins: thread t < nb owns bin nb-1-t; the inclusive scan
// over t counts the candidates in bins at or above it, and the first t where that reaches
// need holds the bin of the need-th largest candidate. Returns the bin; need and ncand
// become the rank within the bin and the bin's count.
__device__ __forceinline__ uint32_t sel_finish8(const SelLds& S, uint32_t nb, int& need, int& ncand) {
  const int tid = tid_opaque(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __syncthreads();
  uint32_t cnt = 0u;
  const int bn = (int)nb - 1 - tid;
  if (tid < 256 && bn >= 0) {
    uint32_t hv[NWAVES];   // every row read before the clears (a read after a clear waits for it)
#pragma unroll
    for (int w = 0; w < NWAVES; w++) hv[w] = S.hist[w * 256 + bn];
#pragma unroll
    for (int w = 0; w < NWAVES; w++) {
      cnt += hv[w];
      S.hist[w * 256 + bn] = 0u;
    }
  }
  const uint32_t x = wave_incl_scan_u32(cnt);
  if (lane == 63 && wave < 4) S.wsum[wave] = x;
  __syncthreads();
  uint32_t cum = x;
  for (int w = 0; w < wave && w < 4; w++) cum += S.wsum[w];
  const bool hit = tid < 256 && bn >= 0 && cum >= (uint32_t)need;
  const uint64_t m = __ballot(hit);
  if (wave < 4 && lane == 0) S.tot[wave] = m ? (uint32_t)(wave * 64 + __ffsll((unsigned long long)m) - 1) : 0xffffffffu;
  if (hit && (uint32_t)tid == (m ? (uint32_t)(wave * 64 + __ffsll((unsigned long long)m) - 1) : 0xffffffffu)) {
    S.sv[4 + wave] = (uint32_t)need - (cum - cnt);   // rank inside the bin
    S.sv[8 + wave] = cnt;
  }
  __syncthreads();
  uint32_t tb = S.tot[0], wb = 0;
  for (int w = 1; w < 4; w++)
    if (S.tot[w] < tb) { tb = S.tot[w]; wb = (uint32_t)w; }
  need = (int)S.sv[4 + wb];
  ncand = (int)S.sv[8 + wb];
  const uint32_t bin = nb - 1u - tb;
  __syncthreads();   // S.tot / S.sv / S.wsum are reused by the next pass
  return bin;
}
// Ranks up to SEL_CMAX candidates (S.chi/clo/ctk[0, nc)) by (key desc, token asc); calls
// taken(c, rank < need) from one lane per candidate.
template <typename F>
__device__ __forceinline__ void sel_rank(const SelLds& S, int nc, int need, F&& taken) {
  const int tid = tid_opaque();
  const int c = tid >> 2, part = tid & 3;
  int rank = 0;
  if (c < nc) {
    const uint32_t h = S.chi[c], l = S.clo[c], t = S.ctk[c];
    // four candidates per trip, loaded together (one LDS round trip each, not per candidate)
    for (int d0 = part; d0 < nc; d0 += 16) {
      uint32_t hd[4], ld[4], td[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int d = min(d0 + 4 * u, nc - 1);
        hd[u] = S.chi[d];
        ld[u] = S.clo[d];
        td[u] = S.ctk[d];
      }
#pragma unroll
      for (int u = 0; u < 4; u++)
        rank += (d0 + 4 * u < nc && (hd[u] > h || (hd[u] == h && (ld[u] > l || (ld[u] == l && td[u] < t))))) ? 1 : 0;
    }
  }
  rank += __shfl_xor(rank, 1, 64);
  rank += __shfl_xor(rank, 2, 64);
  if (c < nc && part == 0) taken(c, rank < need);
}

// Selection over every token (the bound left more candidates than the per-wave lists
// hold): keys reloaded into 68 registers per thread, flags per token in LDS. Kept out of
// line so that its registers do not weigh on the rest of the kernel.
__device__ __noinline__ void sel_all_tokens(const uint32_t* kh, const uint32_t* kl, uint64_t* isel, int T, int K,
                                            uint32_t k1, float* act, double* red) {
  const SelLds S = sel_carve(act);
  const int tid = tid_opaque();
  int need = K, ncand = T;
  uint32_t key[SEL_MAXJ];
#pragma unroll
  for (int j = 0; j < SEL_MAXJ; j++) {
    const int t = tid + j * BLOCK;
    key[j] = t < T ? ld_u32(kh + t) : 0u;
  }
  for (int rr = 0; rr < SEL_ROWS; rr++) S.hist[rr * BLOCK + tid] = 0u;   // passes clear while reducing
  uint32_t pre = 0, pm = 0;
  const uint32_t npad = (uint32_t)(SEL_MAXJ * BLOCK - T);   // padding keys (0): bin 0 while the prefix is 0
  {
    int shift = 32;
    while (ncand > SEL_CMAX && shift > 0) {
      const int wdt = min(5, shift);
      shift -= wdt;
      sel_count<SEL_MAXJ>(S, [&](int j) { return key[j]; }, [&](int j) { return (key[j] & pm) == pre; }, shift,
                          (1u << wdt) - 1u);
      const uint32_t b = sel_finish_pass(S, 1u << wdt, pre == 0u ? npad : 0u, need, ncand);
      pre |= b << shift;
      pm |= ((1u << wdt) - 1u) << shift;
    }
  }
  uint32_t cb0 = 0u, cb1 = 0u, cb2 = 0u;   // candidate bits per column j
#pragma unroll
  for (int j = 0; j < SEL_MAXJ; j++) {   // every column: the contiguous ranges below read them all
    const uint32_t mk = key[j] & pm;
    const bool cand = key[j] != 0u && mk == pre;
    S.fl[tid + j * BLOCK] = (uint8_t)((key[j] != 0u && mk > pre ? 1u : 0u) | (cand ? 2u : 0u));
    const uint32_t bt = (uint32_t)cand << (j & 31);
    if (j < 32) cb0 |= bt;
    else if (j < 64) cb1 |= bt;
    else cb2 |= bt;
  }
  auto cbit = [&](int j) -> bool { return ((j < 32 ? cb0 : j < 64 ? cb1 : cb2) >> (j & 31)) & 1u; };
  if (ncand > SEL_CMAX) {
    // the candidates share all 32 high bits: the same passes over the low halves
    uint32_t lo[SEL_MAXJ];
#pragma unroll
    for (int j = 0; j < SEL_MAXJ; j++) lo[j] = cbit(j) ? ld_u32(kl + tid + j * BLOCK) : 0u;
    uint32_t lpre = 0, lpm = 0;
    int shift = 32;
    while (ncand > SEL_CMAX && shift > 0) {
      const int wdt = min(5, shift);
      shift -= wdt;
      sel_count<SEL_MAXJ>(S, [&](int j) { return lo[j]; }, [&](int j) { return cbit(j) && (lo[j] & lpm) == lpre; },
                          shift, (1u << wdt) - 1u);
      const uint32_t b = sel_finish_pass(S, 1u << wdt, 0u, need, ncand);
      lpre |= b << shift;
      lpm |= ((1u << wdt) - 1u) << shift;
    }
    int cut = T;   // fully equal keys beyond SEL_CMAX: the `need` lowest indices, cut found by bisection
    if (ncand > SEL_CMAX) {
      int lo_m = 0, hi_m = T;
      while (lo_m < hi_m) {
        const int mid = (lo_m + hi_m) >> 1;
        int c = 0;
#pragma unroll
        for (int j = 0; j < SEL_MAXJ; j++) c += (cbit(j) && (lo[j] & lpm) == lpre && tid + j * BLOCK < mid) ? 1 : 0;
        const double tc = block_sum((double)c, red);
        if (tc >= (double)need) hi_m = mid;
        else lo_m = mid + 1;
      }
      cut = lo_m;
      ncand = 0;
    }
#pragma unroll
    for (int j = 0; j < SEL_MAXJ; j++) {
      if (cbit(j)) {
        const uint32_t mk = lo[j] & lpm;
        const int t = tid + j * BLOCK;
        S.fl[t] = (uint8_t)(mk > lpre || (mk == lpre && ncand == 0 && t < cut) ? 1u
                            : (mk == lpre && ncand > 0) ? 2u : 0u);
      }
    }
  }
  __syncthreads();
  // this thread's contiguous token range [r0, r0 + SEL_MAXJ) of the flags
  const int r0 = tid * SEL_MAXJ;
  auto load_range = [&](uint32_t* wds) {
#pragma unroll
    for (int q = 0; q < SEL_MAXJ / 4; q++) wds[q] = reinterpret_cast<const uint32_t*>(S.fl + r0)[q];
  };
  if (ncand > 0) {
    uint32_t wds[SEL_MAXJ / 4];
    load_range(wds);
    uint32_t cn = 0;
#pragma unroll
    for (int q = 0; q < SEL_MAXJ / 4; q++) cn += __popc((wds[q] >> 1) & 0x01010101u);
    uint32_t o = block_excl_scan(cn, S.wsum);
#pragma unroll
    for (int q = 0; q < SEL_MAXJ / 4; q++) {
      uint32_t m = (wds[q] >> 1) & 0x01010101u;
      while (m) {
        const int b = __ffs(m) - 1;
        m &= m - 1u;
        if (o < (uint32_t)SEL_CMAX) S.ctk[o] = (uint32_t)(r0 + 4 * q + (b >> 3));
        o++;
      }
    }
    __syncthreads();
    const int nc = min(ncand, SEL_CMAX);
    if (tid < nc) {
      S.chi[tid] = ld_u32(kh + S.ctk[tid]);
      S.clo[tid] = ld_u32(kl + S.ctk[tid]);
    }
    __syncthreads();
    sel_rank(S, nc, need, [&](int c, bool tk) { S.fl[S.ctk[c]] = tk ? 1 : 0; });
    __syncthreads();
  }
  {
    uint32_t wds[SEL_MAXJ / 4];
    load_range(wds);
    uint32_t cn = 0;
#pragma unroll
    for (int q = 0; q < SEL_MAXJ / 4; q++) cn += __popc(wds[q] & 0x01010101u);
    uint32_t o = block_excl_scan(cn, S.wsum);
#pragma unroll
    for (int q = 0; q < SEL_MAXJ / 4; q++) {
      uint32_t m = wds[q] & 0x01010101u;
      while (m) {
        const int b = __ffs(m) - 1;
        m &= m - 1u;
        if (o < (uint32_t)K) S.hist[o] = (uint32_t)(r0 + 4 * q + (b >> 3));
        o++;
      }
    }
  }
  sel_write_out(S, isel, K, k1);
}

// Everything the selecting workgroup needs, passed by value to the out-of-line selection.
struct SelArgs {
  uint64_t* isel;
  const uint32_t* kh;      // [T] key high halves (all-token path)
  const uint32_t* kl;      // [T] key low halves
  const uint64_t* ilist;   // [nwg][SEL_LIST] LL words: each scorer's top key high halves, rank order
  const uint32_t* ilo;     // [nwg][SEL_LIST] their low halves
  const uint32_t* itok;    // [nwg][SEL_LIST] their tokens
  uint32_t* status;
  long long budget;
  int nwg, layer, token, w, T, K;
  uint32_t k1;
  int red_off, tr_off;   // float offsets of L.red and L.tr from the LDS base (L.act is the base)
  int tron;              // device trace on for this step
};

// A pointer that arrived in vector registers (an out-of-line call's argument) made
// wave-uniform, so that loads through it take the scalar-base + vector-offset form.
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}

// The selection proper (the selecting workgroup, T > K), kept out of line: its registers
// and constants stay inside this function instead of weighing on the whole kernel.
// Returns 0 when a wait expired or another workgroup aborted.
__device__ __noinline__ int sel_select(SelArgs sa) {
  extern __shared__ float lds_raw[];
  float* act = lds_raw;
  double* red = reinterpret_cast<double*>(lds_raw + sa.red_off);
  uint64_t* tr = reinterpret_cast<uint64_t*>(lds_raw + sa.tr_off);
  Ctx cx;
  cx.budget = sa.budget;
  cx.w = sa.w;
  cx.nwg = sa.nwg;
  cx.status = sa.status;
  cx.layer = sa.layer;
  cx.token = sa.token;
  const uint32_t k1 = sa.k1;
  const int tid = tid_opaque(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = sa.T, K = sa.K, nwg = cx.nwg, NE = nwg * SEL_LIST;
  uint64_t* isel = sa.isel;
  auto stp = [&](int slot) {
    if (sa.tron && tid_opaque() == 0) tr[slot] = wall_clock64();
  };
  const SelLds S = sel_carve(act);
  // a taken token's bit, set where the entry is decided
  auto take = [&](uint32_t t) {
    __hip_atomic_fetch_or(lds_ptr(&S.bm[t >> 5]), 1u << (t & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  stp(47);
  // every scorer's list, one word per thread and slot
  if (!ll_fetch<SEL_EPT>(cx, S.lst, sa.ilist, NE, k1, W_ILIST)) return 0;
  stp(46);
  // the bound: the smallest of the scorers' r-th keys (0 when a scorer holds fewer than r)
  {
    const int r = (K + nwg - 1) / nwg;
    uint32_t b = 0xffffffffu;
    if (tid < nwg) b = r <= SEL_LIST ? S.lst[tid * SEL_LIST + r - 1] : 0u;
    b = wave_minmax_u32<false>(b);
    if (lane == 0) S.tot[wave] = b;
    for (int i = tid; i < SEL_BMW * BLOCK; i += BLOCK) S.bm[i] = 0u;
    for (int rr = 0; rr < SEL_ROWS; rr++) S.hist[rr * BLOCK + tid] = 0u;   // passes clear while reducing
  }
  __syncthreads();
  uint32_t lb = S.tot[0];
  for (int i = 1; i < NWAVES; i++) lb = min(lb, S.tot[i]);
  // ---- entries e = tid + q*BLOCK; valid when a key (nonzero) reaches the bound
  // (entries past NE read the last one, unconditionally: no per-load branch; they are
  // never valid, so their tokens and low halves are never used)
  const uint32_t* itok = uniform_ptr(sa.itok);
  const uint32_t* ilo = uniform_ptr(sa.ilo);
  uint32_t etk[SEL_EPT];   // their tokens, in flight during the passes (used for the taken ones)
#pragma unroll
  for (int q = 0; q < SEL_EPT; q++) etk[q] = ld_u32_off(itok, (uint32_t)min(tid + q * BLOCK, NE - 1) * 4u);
  uint32_t elo[SEL_EPT];   // and their low halves (ranking and ties)
#pragma unroll
  for (int q = 0; q < SEL_EPT; q++) elo[q] = ld_u32_off(ilo, (uint32_t)min(tid + q * BLOCK, NE - 1) * 4u);
  uint32_t eh[SEL_EPT];
  uint32_t ev = 0u, cn = 0u, mx = 0u, mn = 0xffffffffu;
#pragma unroll
  for (int q = 0; q < SEL_EPT; q++) {
    const int e = tid + q * BLOCK;
    const uint32_t hr = S.lst[min(e, NE - 1)];
    const uint32_t h = e < NE ? hr : 0u;
    const bool v = h != 0u && h >= lb;
    eh[q] = v ? h : 0u;
    ev |= (uint32_t)v << q;   // (shift form: a literal mask would be hoisted into a register)
    cn += v ? 1u : 0u;
    mx = v ? max(mx, h) : mx;
    mn = v ? min(mn, h) : mn;
  }
  // the lists are complete when no scorer holds an unlisted key whose high half reaches
  // the bound (its unlisted keys are at most its last listed one)
  const int ntw = tid < T ? (T - 1 - tid) / nwg + 1 : 0;
  uint32_t miss = (tid < nwg && ntw > SEL_LIST && S.lst[tid * SEL_LIST + SEL_LIST - 1] >= lb) ? 1u : 0u;
  cn = wave_sum_u32(cn);
  mx = wave_minmax_u32<true>(mx);
  mn = wave_minmax_u32<false>(mn);
  miss = wave_minmax_u32<true>(miss);
  if (lane == 0) {
    S.wsum[wave] = cn;
    S.wsum[8 + wave] = mx;
    S.wsum[16 + wave] = mn;
    S.wsum[24 + wave] = miss;
  }
  __syncthreads();
  uint32_t C = 0u, X = 0u, N = 0xffffffffu, M = 0u;
  for (int i = 0; i < NWAVES; i++) {
    C += S.wsum[i];
    X = max(X, S.wsum[8 + i]);
    N = min(N, S.wsum[16 + i]);
    M |= S.wsum[24 + i];
  }
  if (M) {   // keys beyond the lists can be chosen: every token
    stp(TR_SEL_KEYS);
    sel_all_tokens(sa.kh, sa.kl, isel, T, K, k1, act, red);
    stp(TR_SEL_DONE);
    return 1;
  }
  stp(TR_SEL_KEYS);
  const uint32_t dif = X ^ N;
  const int common = dif ? __clz(dif) : 32;   // leading bits every valid entry shares
  uint32_t pm = common >= 32 ? 0xffffffffu : ~(0xffffffffu >> common);
  uint32_t pre = X & pm;
  int need = K, ncand = (int)C;
  int shift = 32 - common, npass = 0;
  while (ncand > SEL_CMAX && shift > 0) {
    const int wdt = min(8, shift);
    shift -= wdt;
    sel_count8<SEL_EPT>(S, [&](int q) { return eh[q]; }, [&](int q) { return (ev >> q & 1u) && (eh[q] & pm) == pre; },
                        shift, (1u << wdt) - 1u);
    const uint32_t b = sel_finish8(S, 1u << wdt, need, ncand);
    pre |= b << shift;
    pm |= ((1u << wdt) - 1u) << shift;
    stp(39 + min(npass++, 5));
  }
  uint32_t ecb = 0u;   // candidate bits per entry column
#pragma unroll
  for (int q = 0; q < SEL_EPT; q++) {
    const uint32_t mk = eh[q] & pm;
    const bool v = ev >> q & 1u;
    if (v && mk > pre) take(etk[q]);
    ecb |= (uint32_t)(v && mk == pre) << q;
  }
  uint32_t pend = ecb;   // entries still undecided (to be ranked)
  if (ncand > SEL_CMAX) {
    // ---- the candidates share the whole high half: the low halves, then the token order
    uint32_t lpre = 0, lpm = 0;
    int ls = 32;
    while (ncand > SEL_CMAX && ls > 0) {
      const int wdt = min(8, ls);
      ls -= wdt;
      sel_count8<SEL_EPT>(S, [&](int q) { return elo[q]; },
                          [&](int q) { return (ecb >> q & 1u) && (elo[q] & lpm) == lpre; }, ls, (1u << wdt) - 1u);
      const uint32_t b = sel_finish8(S, 1u << wdt, need, ncand);
      lpre |= b << ls;
      lpm |= ((1u << wdt) - 1u) << ls;
    }
    int cut = 0;
    if (ncand > SEL_CMAX) {   // equal 64-bit keys: the `need` lowest tokens, cut found by bisection
      int lo_m = 0, hi_m = T;
      while (lo_m < hi_m) {
        const int mid = (lo_m + hi_m) >> 1;
        int c = 0;
#pragma unroll
        for (int q = 0; q < SEL_EPT; q++)
          c += ((ecb >> q & 1u) && (elo[q] & lpm) == lpre && etk[q] < (uint32_t)mid) ? 1 : 0;
        const double tc = block_sum((double)c, red);
        if (tc >= (double)need) hi_m = mid;
        else lo_m = mid + 1;
      }
      cut = lo_m;
      ncand = 0;
    }
    pend = 0u;
#pragma unroll
    for (int q = 0; q < SEL_EPT; q++) {
      if (ecb >> q & 1u) {
        const uint32_t mk = elo[q] & lpm;
        if (mk > lpre || (mk == lpre && ncand == 0 && etk[q] < (uint32_t)cut)) take(etk[q]);
        pend |= (uint32_t)(mk == lpre && ncand > 0) << q;
      }
    }
  }
  if (ncand > 0) {
    // ---- at most SEL_CMAX undecided entries: their owners write them (hi, lo, token) to
    // the rank arrays in thread order, at offsets from a scan of their counts (the ranking
    // does not depend on the order; one counter bumped per entry serialized its owners)
    uint32_t o = block_excl_scan((uint32_t)__popc(pend), S.wsum);
#pragma unroll
    for (int q = 0; q < SEL_EPT; q++) {
      if (pend >> q & 1u) {
        if (o < (uint32_t)SEL_CMAX) {
          S.chi[o] = eh[q];
          S.clo[o] = elo[q];
          S.ctk[o] = etk[q];
        }
        o++;
      }
    }
    __syncthreads();
    const int nc = min(ncand, SEL_CMAX);
    stp(45);
    sel_rank(S, nc, need, [&](int c, bool tk) {
      if (tk) take(S.ctk[c]);
    });
  }
  // ---- the token bitmap is complete: the output in ascending token order
  __syncthreads();
  stp(TR_SEL_PASSES);
  {
    uint32_t bw[SEL_BMW];
    uint32_t nb = 0;
#pragma unroll
    for (int q = 0; q < SEL_BMW; q++) {
      bw[q] = S.bm[tid * SEL_BMW + q];
      nb += __popc(bw[q]);
    }
    uint32_t o = block_excl_scan(nb, S.wsum);
#pragma unroll
    for (int q = 0; q < SEL_BMW; q++) {
      uint32_t m = bw[q];
      while (m) {
        const int b = __ffs(m) - 1;
        m &= m - 1u;
        if (o < (uint32_t)K) S.hist[o] = (uint32_t)((tid * SEL_BMW + q) * 32 + b);
        o++;
      }
    }
  }
  sel_write_out(S, isel, K, k1);
  stp(TR_SEL_DONE);
  return 1;
}

template <class SH>
__device__ __forceinline__ bool stage_sel_mla(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  if (cx.w != SEL_WG) return true;
  const int T = st.pos + 1, K = min(a.c.itopk, T);
  uint64_t* isel = wsp<uint64_t>(a, a.off.isel);
  if (T <= K) {   // every token
    for (int j = tid_opaque(); j < T; j += BLOCK) ll_put(isel + j, (uint32_t)j, st.k1);
    stamp(a, cx, st, TR_SEL_DONE);
    return true;
  }
  SelArgs sa;
  sa.isel = isel;
  sa.kh = wsp<uint32_t>(a, a.off.ikh);
  sa.kl = wsp<uint32_t>(a, a.off.ikl);
  sa.ilist = wsp<uint64_t>(a, a.off.ilist);
  sa.ilo = wsp<uint32_t>(a, a.off.ilo);
  sa.itok = wsp<uint32_t>(a, a.off.itok);
  sa.status = cx.status;
  sa.budget = cx.budget;
  sa.nwg = cx.nwg;
  sa.layer = cx.layer;
  sa.token = cx.token;
  sa.w = cx.w;
  sa.T = T;
  sa.K = K;
  sa.k1 = st.k1;
  sa.red_off = (int)(reinterpret_cast<float*>(L.red) - L.act);
  sa.tr_off = (int)(reinterpret_cast<float*>(L.tr) - L.act);
  sa.tron = (a.trace && st.idx < a.trace_steps) ? 1 : 0;
  return sel_select(sa) != 0;
}

// ------------------------------------------------------------------ ABS: q_lat_h = W_UK_h^T q_nope_h
// Workgroup w owns cpw consecutive outputs of head h: columns [c0, c0 + cpw) of the head's
// [nope x kv_lora] block of W_UK (for FP8 this is one 128x128 scale block). Each thread
// streams one 16-byte chunk of several rows; the per-thread partial sums over rows are
// added across row groups in LDS in a fixed order.
template <class SH>
__device__ __forceinline__ bool stage_absorb_mla(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  constexpr int EPC = SH::FP8 ? 16 : 8, ESZ = SH::FP8 ? 1 : 2;
  constexpr int SBK = (SH::KL + 127) / 128;
  const int cpw = c.cpw;
  const int h = (cx.w * cpw) / SH::KL, c0 = (cx.w * cpw) % SH::KL;
  const int cpr = cpw / EPC;            // 16-byte chunks per row (host: cpw % EPC == 0, BLOCK % cpr == 0)
  const int rpp = BLOCK / cpr;          // rows per pass
  constexpr int MAXP = 4;               // passes over the ND rows (host: ND <= MAXP * rpp)
  const int tid = tid_opaque();
  const int ck = tid % cpr, rr = tid / cpr;
  uint4 wv[MAXP];
  float sc[MAXP];
#pragma unroll
  for (int p = 0; p < MAXP; p++) {
    wv[p] = make_uint4(0u, 0u, 0u, 0u);
    sc[p] = 0.f;
    if (p * rpp < SH::ND) {   // uniform: only the passes the head needs
      const int d = min(rr + p * rpp, SH::ND - 1);
      const size_t row = (size_t)h * SH::ND + d;
      wv[p] = ld_stream16(Ly.w_uk.w + (row * SH::KL + c0 + ck * EPC) * ESZ);
      sc[p] = SH::FP8 ? gp(Ly.w_uk.s)[(row >> 7) * SBK + ((c0 + ck * EPC) >> 7)] : 1.f;
    }
  }
  float* qv = L.act;                    // [ND] q_nope of head h
  const int rs = rpp + 1;               // column stride of red (padded: spreads the stores over the banks)
  float* red = L.act + SH::ND;          // [cpw][rs] per-thread partial sums, column-major
  float* red2 = red + cpw * rs;         // [BLOCK / cpw][cpw] sums of row groups, then [cpw] totals
  if (!ll_fetch<per_for(SH::ND)>(cx, reinterpret_cast<uint32_t*>(qv), wsp<uint64_t>(a, a.off.q) + (size_t)h * SH::ND,
                                 SH::ND, st.k1, W_QN))
    return false;
  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; e++) acc[e] = 0.f;
#pragma unroll
  for (int p = 0; p < MAXP; p++) {
    const int d = rr + p * rpp;
    if (p * rpp < SH::ND) {
      const float q = d < SH::ND ? qv[d] * sc[p] : 0.f;
      const uint32_t wd[4] = {wv[p].x, wv[p].y, wv[p].z, wv[p].w};
      if constexpr (SH::FP8) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[i], false);
          const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[i], true);
          acc[4 * i + 0] = fmaf(lo.x, q, acc[4 * i + 0]);
          acc[4 * i + 1] = fmaf(lo.y, q, acc[4 * i + 1]);
          acc[4 * i + 2] = fmaf(hi.x, q, acc[4 * i + 2]);
          acc[4 * i + 3] = fmaf(hi.y, q, acc[4 * i + 3]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          acc[2 * i] = fmaf(bf_lo(wd[i]), q, acc[2 * i]);
          acc[2 * i + 1] = fmaf(bf_hi(wd[i]), q, acc[2 * i + 1]);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EPC; e++) red[(ck * EPC + e) * rs + rr] = acc[e];
  __syncthreads();
  // column sums over the rpp row partials, all threads at once: thread t adds the rows
  // [gq * rpg, (gq + 1) * rpg) of column t % cpw (four independent chains), then the
  // BLOCK / cpw group sums of a column are added in group order
  {
    const int ng = BLOCK / cpw, rpg = rpp / ng;   // host: cpw divides BLOCK (so ng divides rpp)
    const int j = tid % cpw, gq = tid / cpw;
    const float* col = red + j * rs + gq * rpg;
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
    int g = 0;
    for (; g + 4 <= rpg; g += 4) {
#pragma unroll
      for (int u = 0; u < 4; u++) s4[u] += col[g + u];
    }
    for (; g < rpg; g++) s4[0] += col[g];
    red2[gq * cpw + j] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    __syncthreads();
    float tot = 0.f;
    if (tid < cpw)
      for (int q = 0; q < ng; q++) tot += red2[q * cpw + tid];
    __syncthreads();
    if (tid < cpw) red2[tid] = tot;
    __syncthreads();
  }
  // q_lat as bf16 pairs: the attention's matrix cores take it in bf16 (same rounding)
  uint64_t* ql = wsp<uint64_t>(a, a.off.qlat) + ((size_t)h * SH::KL + c0) / 2;
  for (int j = 2 * tid; j < cpw; j += 2 * BLOCK)
    ll_put(ql + j / 2, f32_to_bf16(red2[j]) | (f32_to_bf16(red2[j + 1]) << 16), st.k1);
  __syncthreads();
  stamp(a, cx, st, TR_ATT_SCORES);
  return true;
}

// ------------------------------------------------------------------ ATT: flash-decoding over the latent cache
// Workgroup w = (head group hg, chunk ch) with ch = w % nch: the nch chunk workgroups of a
// head group sit on the XCDs in turn, and the workgroups of one chunk share an XCD (w % 8
// is the same), so a chunk's latent rows come from HBM once and from L2 after that.
// Per 32-row sub-block: rows staged in LDS (double buffer, next block's loads in flight
// during the products), S = Q . C^T with the 36 k-steps split over 4 wave pairs, online
// softmax (wave h owns head h), O += P . C[:, :kv_lora] with each wave owning 64 columns.
// Q and P are rounded to bf16 for the matrix cores; scores, softmax and O stay fp32.
template <class SH>
__device__ __forceinline__ bool stage_attn_mla(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  const uint32_t k1 = st.k1;
  constexpr int LAT = SH::LAT, KL = SH::KL, RD = SH::RD, HPW = SH::HPW, TB = SH::TB, CSTR = SH::CSTR;
  constexpr int KSTEPS = LAT / 16, KQ = KSTEPS / 4;   // k-steps per wave pair
  constexpr int CPRW = LAT / 8;                        // 16-byte chunks per latent row
  constexpr int NLD = (TB * CPRW + BLOCK - 1) / BLOCK; // staging loads per thread per sub-block
  static_assert(KSTEPS % 4 == 0 && KL == 512 && (HPW == NWAVES || HPW == 2 * NWAVES) && TB == 32, "attention tiling");
  constexpr int HS = HPW / NWAVES;   // heads per wave: one, or one per 32-lane half
  // the head this lane's softmax state belongs to
  const int hown = (tid_opaque() >> 6) * HS + (HS == 2 ? ((tid_opaque() & 63) >> 5) : 0);
  const int tid = tid_opaque();
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = c.cpg;
  const int hg = cx.w / nch, ch = cx.w % nch;
  const int hbase = hg * HPW;
  const int pos = st.pos, T = pos + 1;
  // the last chunk's new row: this thread's RMSNorm weights (c_kv) or RoPE factors (k_rope),
  // loaded before the latent rows so that they do not queue behind them
  float nw0 = 0.f, nw1 = 0.f;
  if (ch == nch - 1 && tid_opaque() < LAT / 2) {
    const int k = 2 * tid_opaque();
    const PLD_GLOBAL float* src = k < KL ? gp(Ly.kv_norm) + k : gp(wsp<float>(a, a.off.rope)) + (size_t)pos * RD + (k - KL);
    nw0 = src[0];
    nw1 = src[1];
  }
  // dense: the chunk's rows are [t0, t1) of the T - 1 history rows (the row of position pos
  // is added by the last chunk after its blocks); sparse: entries [t0, t1) of the
  // indexer's ascending list of K selected rows (the new row, if chosen, is the last)
  const int K = SH::SPARSE ? min(c.itopk, T) : T - 1;
  const int t0 = split_at(K, nch, ch), t1 = split_at(K, nch, ch + 1), n = t1 - t0;
  const int fresh = a.pos0;
  const int nst = max(0, min(n, fresh - t0));            // dense: static rows of the chunk: [0, nst)
  const uint16_t* lat = Ly.lat;
  // LDS (inside L.act)
  uint16_t* Qs = reinterpret_cast<uint16_t*>(L.act);     // [16][CSTR] bf16 (rows >= HPW zero)
  uint16_t* Cs = Qs + 16 * CSTR;                          // [2][TB][CSTR] bf16
  uint16_t* Ps = Cs + 2 * TB * CSTR;                      // [16][TB] bf16
  float* Ssc = reinterpret_cast<float*>(Ps + 16 * TB);   // [4][2][256] partial score tiles
  float* alph = Ssc + 4 * 2 * 256;                        // [HPW]
  float* qtmp = reinterpret_cast<float*>(Cs + TB * CSTR); // q staging (Cs buffer 1, free at start)
  uint16_t* newrow = reinterpret_cast<uint16_t*>(alph + 16);   // [LAT] the row of position pos
  float* ntmp = reinterpret_cast<float*>(newrow + LAT);  // [LAT] its fp32 raw values
  int* srows = reinterpret_cast<int*>(ntmp + LAT);        // sparse: [n] rows of this chunk
  // q of the head group: q_lat [HPW][KL] and q_rope [HPW][RD] as bf16 pairs (LL) -> rows of Qs
  auto fetch_q = [&]() -> bool {
    uint32_t* qw = reinterpret_cast<uint32_t*>(qtmp);   // [HPW][KL/2] then [HPW][RD/2] words
    if (!ll_fetch<per_for(HPW * KL / 2)>(cx, qw, wsp<uint64_t>(a, a.off.qlat) + (size_t)hbase * KL / 2, HPW * KL / 2,
                                         k1, W_QLAT))
      return false;
    if (!ll_fetch<per_for(HPW * RD / 2)>(cx, qw + HPW * KL / 2, wsp<uint64_t>(a, a.off.qr) + (size_t)hbase * RD / 2,
                                         HPW * RD / 2, k1, W_QLAT))
      return false;
    static_assert(CSTR % 2 == 0, "Qs rows hold whole bf16 pairs");
    for (int i = tid; i < 16 * LAT / 2; i += BLOCK) {
      const int h = i / (LAT / 2), k2 = i % (LAT / 2);
      const uint32_t v = h >= HPW ? 0u : (k2 < KL / 2 ? qw[h * (KL / 2) + k2] : qw[HPW * KL / 2 + h * (RD / 2) + (k2 - KL / 2)]);
      reinterpret_cast<uint32_t*>(Qs + h * CSTR)[k2] = v;
    }
    return true;
  };
  if constexpr (SH::SPARSE) {
    // the queries were ready long before the selection: fetched first, so that only the
    // selected rows' loads remain once the selection arrives (dense: fetched after the
    // first latent rows are issued, overlapping their latency)
    if (!fetch_q()) return false;
    if (n > 0 && !ll_fetch<1>(cx, reinterpret_cast<uint32_t*>(srows), wsp<uint64_t>(a, a.off.isel) + t0, n, k1,
                              W_ISEL))
      return false;
  }
  auto srow = [&](int t) -> size_t {
    if constexpr (SH::SPARSE) return (size_t)srows[min(t, n - 1)];
    else return (size_t)(nst > 0 ? t0 + min(t, nst - 1) : 0);
  };
  // index inside the chunk of the row of position pos (its bf16 row is patched in from
  // LDS), or -1; the chunk that computes the new row and appends it to the cache
  const int pidx = SH::SPARSE ? ((ch == nch - 1 && n > 0 && srows[n - 1] == pos) ? n - 1 : -1) : -1;
  const bool newrow_here = ch == nch - 1;
  // Staging registers: three sub-blocks in flight (sets A, B, C in turn); chunk i of a
  // block covers (row i / CPRW, chunk i % CPRW). A block's loads are issued DEPTH blocks
  // before it is staged into LDS, so the wait at staging time covers ~3 blocks of work.
  // All loads are unconditional (clamped rows; blocks past the chunk read one uniform
  // address and are masked), so the in-order load waits stay exact. A sub-block that holds
  // rows written inside this launch reads its rows coherently; every other sub-block (in
  // particular the static rows of the same chunk) reads through L2, where the head groups
  // of a chunk share them. Both kinds issue the same number of loads into the same
  // registers. The row of position pos is patched in from LDS after staging.
  constexpr int DEPTH = 3;
  const int nsb = (n + TB - 1) / TB;
  auto fresh_block = [&](int sb) -> bool {   // does sub-block sb hold a row written in this launch?
    const int last = min(sb * TB + TB, n) - 1;
    if (last < 0) return false;
    return SH::SPARSE ? srows[last] >= fresh : t0 + last >= fresh;
  };
  uint4 cb[DEPTH][NLD];
  auto issue_k = [&](int set, int sb, auto coh_tag) {
    constexpr bool COH = decltype(coh_tag)::value;
    const bool live = sb < nsb;
#pragma unroll
    for (int i = 0; i < NLD; i++) {
      const int idx = min(tid + i * BLOCK, TB * CPRW - 1);
      const int r = idx / CPRW, k = idx % CPRW;
      const int t = max(min(sb * TB + r, n - 1), 0);
      const size_t row = (COH && !SH::SPARSE) ? (size_t)(t0 + t) : srow(t);
      const uint16_t* p = live ? lat + row * LAT + k * 8 : lat;
      cb[set][i] = COH ? ld_coh16(p) : ld_g16(p);
    }
  };
  auto issue = [&](int set, int sb) {
    if (sb < nsb && fresh_block(sb)) issue_k(set, sb, std::true_type{});
    else issue_k(set, sb, std::false_type{});
  };
  // registers -> LDS, then the row of pos from LDS (DS operations only)
  auto store = [&](int set, int sb, int buf) {
    uint16_t* C = Cs + buf * TB * CSTR;
#pragma unroll
    for (int i = 0; i < NLD; i++) {
      const int idx = tid + i * BLOCK;
      if (idx < TB * CPRW) {
        const int r = idx / CPRW, k = idx % CPRW;
        uint32_t* d = reinterpret_cast<uint32_t*>(C + r * CSTR + k * 8);
        d[0] = cb[set][i].x; d[1] = cb[set][i].y; d[2] = cb[set][i].z; d[3] = cb[set][i].w;
      }
    }
    const int rp = pidx - sb * TB;   // row of pos inside this block
    if (pidx >= 0 && rp >= 0 && rp < TB) {
      __syncthreads();
      for (int k = tid; k < LAT / 2; k += BLOCK)
        reinterpret_cast<uint32_t*>(C + rp * CSTR)[k] = reinterpret_cast<const uint32_t*>(newrow)[k];
    }
  };
#pragma unroll
  for (int d = 0; d < DEPTH; d++) issue(d, d);
  // the row of position pos: RMSNorm(c_kv') and RoPE(k_r'), bf16 (before the queries: its
  // input was published by the X stage, so this runs while the absorbed queries are produced)
  if (newrow_here) {
    if (!ll_fetch<per_for(LAT)>(cx, reinterpret_cast<uint32_t*>(ntmp), wsp<uint64_t>(a, a.off.ckvr), LAT, k1, W_KV))
      return false;
    double ss = 0.0;
    for (int i = tid; i < KL; i += BLOCK) ss += (double)ntmp[i] * (double)ntmp[i];
    ss = block_sum(ss, L.red);
    const double r = 1.0 / sqrt(ss / (double)KL + c.eps);
    const PLD_GLOBAL float* g = gp(Ly.kv_norm);
    const PLD_GLOBAL float* rope = gp(wsp<float>(a, a.off.rope)) + (size_t)pos * RD;
    for (int i = tid; i < LAT / 2; i += BLOCK) {
      const int k = 2 * i;
      const bool first = i == tid;   // its factors were loaded at the start of the stage
      float v0, v1;
      if (k < KL) {
        v0 = (float)(((double)ntmp[k] * r) * (double)(first ? nw0 : g[k]));
        v1 = (float)(((double)ntmp[k + 1] * r) * (double)(first ? nw1 : g[k + 1]));
      } else {
        const int d = k - KL;
        const float x0 = ntmp[k], x1 = ntmp[k + 1], cs = first ? nw0 : rope[d], sn = first ? nw1 : rope[d + 1];
        v0 = x0 * cs - x1 * sn;
        v1 = x0 * sn + x1 * cs;
      }
      const uint32_t pair = f32_to_bf16(v0) | (f32_to_bf16(v1) << 16);
      reinterpret_cast<uint32_t*>(newrow)[i] = pair;
      if (hg == 0) st_u32(reinterpret_cast<uint32_t*>(Ly.lat + (size_t)pos * LAT) + i, pair);   // cache append
    }
  }
  if constexpr (!SH::SPARSE) {
    if (!fetch_q()) return false;
  }
  for (int i = tid; i < 16 * TB; i += BLOCK) Ps[i] = 0;
  __syncthreads();
  stamp(a, cx, st, TR_ATT_READY);
  const float scale = 1.0f / sqrtf((float)(SH::ND + SH::RD));
  float m_run = -INFINITY, l_run = 0.f;   // of head hown
  f32x4 O[4];
#pragma unroll
  for (int t = 0; t < 4; t++) O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ln = lane & 15, lq = lane >> 4;
  auto block = [&](const uint16_t* C, int tb0) {
    // ---- S partial: wave pair (wave >> 1) covers k-steps [kq*KQ, kq*KQ+KQ), tile nt = wave & 1
    {
      const int nt = wave & 1, kq = wave >> 1;
      // two independent accumulator chains (even / odd k-steps)
      f32x4 s4 = {0.f, 0.f, 0.f, 0.f}, s5 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KQ; kk++) {
        const int k0 = (kq * KQ + kk) * 16 + 4 * lq;
        const bf16x4 av = *reinterpret_cast<const bf16x4*>(Qs + ln * CSTR + k0);
        const bf16x4 bv = *reinterpret_cast<const bf16x4*>(C + (nt * 16 + ln) * CSTR + k0);
        if (kk & 1) s5 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, s5, 0, 0, 0);
        else s4 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, s4, 0, 0, 0);
      }
      s4 += s5;
      float* dst = Ssc + (kq * 2 + nt) * 256;
#pragma unroll
      for (int q = 0; q < 4; q++) dst[(4 * lq + q) * 16 + ln] = s4[q];
    }
    __syncthreads();
    if (tb0 == 0) stamp(a, cx, st, 23);
    // ---- online softmax: head hown; lane t (of its 32-lane half) is token tb0 + t
    {
      const int h = hown, tl = lane & 31;
      const bool act_lane = HS == 2 || lane < TB;
      float s = -INFINITY;
      if (act_lane && tb0 + tl < n) {
        const int nt = tl >> 4, col = tl & 15;
        s = 0.f;
#pragma unroll
        for (int kq = 0; kq < 4; kq++) s += Ssc[(kq * 2 + nt) * 256 + h * 16 + col];
        s *= scale;
      }
      const float mb = HS == 2 ? half_max_dpp(s) : wave_max_dpp(s);
      const float mnew = fmaxf(m_run, mb);
      const float al = m_run == -INFINITY ? 0.f : __expf(m_run - mnew);
      const float p = s == -INFINITY ? 0.f : __expf(s - mnew);
      l_run = l_run * al + (HS == 2 ? half_sum_dpp(p) : wave_sum_dpp(p));
      m_run = mnew;
      if (act_lane) Ps[h * TB + tl] = (uint16_t)bf16_bits(p);
      if (tl == 0 && act_lane) alph[h] = al;
    }
    __syncthreads();
    if (tb0 == 0) stamp(a, cx, st, 28);
    // ---- O = alpha * O + P . C: wave owns columns [wave*64, wave*64 + 64) (4 tiles)
    {
      float fa[4];
#pragma unroll
      for (int q = 0; q < 4; q++) fa[q] = (4 * lq + q) < HPW ? alph[4 * lq + q] : 0.f;
#pragma unroll
      for (int t = 0; t < 4; t++)
#pragma unroll
        for (int q = 0; q < 4; q++) O[t][q] *= fa[q];
#pragma unroll
      for (int ks = 0; ks < TB / 16; ks++) {
        const bf16x4 av = *reinterpret_cast<const bf16x4*>(Ps + ln * TB + ks * 16 + 4 * lq);
#pragma unroll
        for (int t = 0; t < 4; t++) {
          const int col = (wave * 4 + t) * 16 + ln;
          bf16x4 bv;
#pragma unroll
          for (int q = 0; q < 4; q++) bv[q] = (short)C[(ks * 16 + 4 * lq + q) * CSTR + col];
          O[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, O[t], 0, 0, 0);
        }
      }
    }
  };
  // (only the chunk's own sub-blocks are computed; the loads of the sets past the last
  // one read a uniform address and are never staged)
  {
    for (int sb0 = 0; sb0 < nsb; sb0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; d++) {
        const int sb = sb0 + d;
        if (sb >= nsb) break;
        const int tb0 = sb * TB, buf = sb & 1;
        const uint16_t* C = Cs + buf * TB * CSTR;
        store(d, sb, buf);
        __syncthreads();
        if (sb == 0) stamp(a, cx, st, 17);
        issue(d, sb + DEPTH);   // refill this set, DEPTH blocks ahead
        block(C, tb0);
        if (sb == 0) stamp(a, cx, st, 31);
      }
    }
  }
  if constexpr (!SH::SPARSE) {
    // dense: the row of position pos joins the last chunk's online softmax here, on the
    // vector ALU (as a sub-block of its own it would cost a whole block for one row)
    if (newrow_here) {
      float* sn = Ssc;   // [16] scores, [16] alpha, [16] p (the score tiles are free now)
      {
        constexpr int DPJ = LAT / 32;   // dims per lane: 32 lanes per head row
        const int hr = tid >> 5, j = tid & 31;
        float sv = 0.f;
#pragma unroll
        for (int d = 0; d < DPJ; d++)
          sv = fmaf(bf16_to_f32(Qs[hr * CSTR + j * DPJ + d]), bf16_to_f32(newrow[j * DPJ + d]), sv);
        sv = dpp_sum<32>(sv);   // valid in the last lane of each half-wave
        if (j == 31) sn[hr] = sv * scale;
      }
      __syncthreads();
      {
        const float sv = sn[hown];
        const float mnew = fmaxf(m_run, sv);
        const float al = m_run == -INFINITY ? 0.f : __expf(m_run - mnew);
        const float pn = __expf(sv - mnew);
        l_run = l_run * al + pn;
        m_run = mnew;
        if ((lane & 31) == 0 && (HS == 2 || lane == 0)) {
          sn[16 + hown] = al;
          sn[32 + hown] = pn;
        }
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < 4; t++) {
        const float v = bf16_to_f32(newrow[(wave * 4 + t) * 16 + ln]);
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int h = 4 * lq + q;
          if (h < HPW) O[t][q] = O[t][q] * sn[16 + h] + sn[32 + h] * v;
        }
      }
    }
  }
  stamp(a, cx, st, TR_ATT_SOFTMAX);
  // publish the partial of each head: LL words [m, l, spare | acc as fp16 pairs] at
  // ((h * nch) + ch) * PSTR (fp16 keeps the merged result at fp32 accuracy here: the
  // partial sums stay far inside its range, and the error is set by the bf16 P operand)
  constexpr int PSTR = vp_stride<KL>();
  vm_wait();   // the cache row appended above is visible before this workgroup's next publication
  __syncthreads();
  uint64_t* pll = wsp<uint64_t>(a, a.off.part);
  // (m, l) line of head hown: 8 lanes write words 2 j, 2 j + 1 (m, l, then zeros)
  if ((lane & 31) < 8 && (HS == 2 || lane < 8)) {
    const int j = lane & 7;
    uint64_t* p = pll + ((size_t)(hbase + hown) * nch + ch) * PSTR + 2 * j;
    ll_put_f32(p, j == 0 ? m_run : 0.f, k1);
    ll_put_f32(p + 1, j == 0 ? l_run : 0.f, k1);
  }
  // acc of a tile pair (2u, 2u + 1) as 16 consecutive words per head: the even lanes write
  // tile 2u's pairs (columns ln, ln + 1), the odd lanes tile 2u + 1's (ln - 1, ln)
  const bool ev = (ln & 1) == 0;
#pragma unroll
  for (int u = 0; u < 2; u++) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const float a0 = O[2 * u][q], a1 = O[2 * u + 1][q];
      const float n0 = dpp_mov<0xB1, 0xf, false>(a0), n1 = dpp_mov<0xB1, 0xf, false>(a1);   // lane ln ^ 1
      const float lo = ev ? a0 : n1, hi = ev ? n0 : a1;
      const int h = 4 * lq + q;
      if (h < HPW) {
        const uint32_t pr = (uint32_t)__half_as_ushort(__float2half_rn(lo)) |
                            ((uint32_t)__half_as_ushort(__float2half_rn(hi)) << 16);
        const int word = (wave * 4 + 2 * u) * 8 + (ev ? 0 : 8) + (ln >> 1);
        ll_put(pll + ((size_t)(hbase + h) * nch + ch) * PSTR + VP_ACC + word, pr, k1);
      }
    }
  }
  stamp(a, cx, st, TR_ATT_PARTIAL);
  return true;
}

// ------------------------------------------------------------------ MRG: merge the chunk partials of one head
template <class SH>
__device__ __forceinline__ bool stage_merge_mla(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const KCfg& c = a.c;
  constexpr int KL = SH::KL;
  const int nch = c.cpg, cpw = c.cpw;
  const int h = (cx.w * cpw) / KL, c0 = (cx.w * cpw) % KL;
  const int tid = tid_opaque();
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int PSTR = vp_stride<KL>();
  const int cpw2 = cpw / 2;             // fp16-pair words per chunk
  const int nacc = nch * cpw;           // floats
  const int naw = nch * cpw2;           // their words
  auto pidx = [=](int i) -> int {
    if (i < naw) return (h * nch + i / cpw2) * PSTR + VP_ACC + c0 / 2 + i % cpw2;
    const int j = i - naw;
    return (h * nch + (j >> 1)) * PSTR + (j & 1);
  };
  // word i < naw: the fp16 pair of chunk i / cpw2 at columns 2 (i % cpw2), +1 -> floats 2i, 2i + 1;
  // then the (m, l) words after the nacc floats
  struct StMerge {
    int naw;
    __device__ __forceinline__ void operator()(uint32_t* dst, int i, uint32_t v) const {
      if (i < naw) {
        reinterpret_cast<float2*>(dst)[i] = make_float2(__half2float(__ushort_as_half((unsigned short)(v & 0xffffu))),
                                                         __half2float(__ushort_as_half((unsigned short)(v >> 16))));
      } else {
        dst[naw + i] = v;
      }
    }
  };
  float* accs = L.act;              // [nch][cpw]
  float* mls = L.act + nacc;        // [nch][2]
  float* fw = mls + 2 * nch;        // [nch]
  float* lsum = fw + nch;           // [1]
  float* part = lsum + 1;           // [BLOCK] partial sums over chunk subsets
  stamp(a, cx, st, TR_MERGE_START);
  // one round of loads covers up to 9 * BLOCK words (64 chunks x 64 fp16-pair words + their m, l)
  if (!ll_fetch<9>(cx, reinterpret_cast<uint32_t*>(L.act), wsp<uint64_t>(a, a.off.part), naw + 2 * nch, st.k1,
                   W_PART, pidx, StMerge{naw}))
    return false;
  stamp(a, cx, st, TR_MERGE_COPIED);
  if (wave == 0) {
    float M = -INFINITY;
    for (int cc = lane; cc < nch; cc += 64)
      if (mls[2 * cc + 1] > 0.f) M = fmaxf(M, mls[2 * cc]);
    M = wave_max_dpp(M);
    float ls = 0.f;
    for (int cc = lane; cc < nch; cc += 64) {
      const float l = mls[2 * cc + 1];
      const float f = l > 0.f ? __expf(mls[2 * cc] - M) : 0.f;
      fw[cc] = f;
      ls += f * l;
    }
    ls = wave_sum_dpp(ls);
    if (lane == 0) lsum[0] = ls;
  }
  __syncthreads();
  // column j: np = BLOCK / cpw threads each sum the chunks cc = q, q + np, ... (q = tid / cpw),
  // then thread j adds the np partial sums in order
  const int np = BLOCK / cpw;   // host: cpw divides BLOCK
  {
    const int j = tid % cpw, q = tid / cpw;
    float o = 0.f;
    for (int cc = q; cc < nch; cc += np) o = fmaf(fw[cc], accs[cc * cpw + j], o);
    part[tid] = o;
  }
  __syncthreads();
  uint64_t* ol = wsp<uint64_t>(a, a.off.olat) + (size_t)h * KL + c0;
  if (tid < cpw) {
    float o = 0.f;
    for (int q = 0; q < np; q++) o += part[q * cpw + tid];
    ll_put_f32(ol + tid, o / lsum[0], st.k1);
  }
  stamp(a, cx, st, TR_ATT_MERGED);
  return true;
}

// ------------------------------------------------------------------ UV: o_h = W_UV_h o_lat_h
template <class SH>
__device__ __forceinline__ bool stage_uv_mla(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const DLayer Ly = *gp(st.Ly);
  constexpr int R = SH::NH * SH::VD;
  constexpr size_t RB = (size_t)SH::KL * (SH::FP8 ? 1 : 2);
  const int r0 = split_at(R, cx.nwg, cx.w), r1 = split_at(R, cx.nwg, cx.w + 1);
  const int h = r0 / SH::VD;   // host: every workgroup's rows lie in one head
  bool pending = true;
  auto pre = [&]() -> bool {
    if (!pending) return true;
    pending = false;
    if (!ll_fetch<per_for(SH::KL)>(cx, reinterpret_cast<uint32_t*>(L.act),
                                   wsp<uint64_t>(a, a.off.olat) + (size_t)h * SH::KL, SH::KL, st.k1, W_OLAT,
                                   IdxLinear{}, StPad<SH::FP8>{}))
      return false;
    return true;
  };
  seg_begin();
  seg_set(L, 0, Ly.w_uv.w + (size_t)r0 * RB, Ly.w_uv.s, r1 - r0, r0, 0, 1.f);
  seg_end();
  if (!gemv_list<SH::FP8, SH::KL, PLD_IF_WO>(L.segs, r1 > r0 ? 1 : 0, L.act, L.outb, OUT_STORE, pre)) return false;
  if (!pre()) return false;
  __syncthreads();
  uint64_t* o = wsp<uint64_t>(a, a.off.o);
  for (int r = r0 + tid_opaque(); r < r1; r += BLOCK) ll_put_f32(o + r, L.outb[r - r0], st.k1);
  stamp(a, cx, st, TR_ATT_DONE);
  return true;
}

template <class SH>
__global__ void __launch_bounds__(BLOCK, 1) k_decode_mla(KArgs a) {
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
  // verify (a.drafts set): position t > 0 is fed draft t-1 instead of the argmax; greedy
  // acceptance counts the leading drafts that equal the argmax of the position before
  int accepted = 0;
  bool accepting = true;
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
      // the launch geometry as per-step values: row splits and pass counts derived from
      // it are then computed inside the step instead of being hoisted to kernel entry,
      // where they would hold scalar registers (and spill) across every stage
      Ctx cs = cx;
      asm volatile("" : "+s"(cs.w), "+s"(cs.nwg), "+s"(as.c.cpw), "+s"(as.c.cpg), "+s"(as.c.itopk));
      uint32_t lds0 = 0;
      asm volatile("" : "+s"(lds0));
      Lds L = carve(lds_raw + lds0, a.c);
      st.tr = L.tr;
      cs.wacc = (a.trace && st.idx < a.trace_steps) ? L.tr + TR_WAIT : nullptr;
      stamp(as, cs, st, TR_START);
      PLD_TEST_DELAY(a, cs.w, st.idx, 0);
      if (!stage_x_mla<SH>(cs, as, st, L)) return;
      if (!stage_q_mla<SH>(cs, as, st, L)) return;
      if constexpr (SH::SPARSE) {
        if (!stage_idx_mla<SH>(cs, as, st, L)) return;
      }
      if constexpr (SH::SPARSE) {
        // the selecting workgroup goes straight from its scores to the selection (it is the
        // critical path: every attention workgroup waits for it); its share of the absorbed
        // queries is done by the last workgroup after that one's own share
        const int nabs = cs.w == SEL_WG ? 0 : (cs.w == cs.nwg - 1 ? 2 : 1);
        for (int pass = 0; pass < nabs; pass++) {
          Ctx ca = cs;
          int wsel = SEL_WG;
          asm volatile("" : "+s"(wsel));
          ca.w = pass == 0 ? cs.w : wsel;
          if (!stage_absorb_mla<SH>(ca, as, st, L)) return;
        }
        if (!stage_sel_mla<SH>(cs, as, st, L)) return;
      } else {
        if (!stage_absorb_mla<SH>(cs, as, st, L)) return;
      }
      PLD_TEST_DELAY(a, cs.w, st.idx, 1);
      if (!stage_attn_mla<SH>(cs, as, st, L)) return;
      if (!stage_merge_mla<SH>(cs, as, st, L)) return;
      if (!stage_uv_mla<SH>(cs, as, st, L)) return;
      if (!stage_wo<SH>(cs, as, st, L)) return;
      PLD_TEST_DELAY(a, cs.w, st.idx, 2);
      if (!stage_ffn<SH>(cs, as, st, L)) return;
      PLD_TEST_DELAY(a, cs.w, st.idx, 3);
      if (!stage_down<SH>(cs, as, st, L, last ? as.out_hidden : nullptr)) return;
      if constexpr (SH::FP8) {
        if (a.head_on && li == a.n_layers - 1) {
          if (!stage_head<SH>(cs, as, st, L, t, &token)) return;
          if (a.drafts && t + 1 < a.n_tokens) {
            const int d = gp(a.drafts)[t];   // caller's draft for position t + 1
            accepting = accepting && d == token;
            accepted += accepting ? 1 : 0;
            token = min(max(d, 0), a.c.vocab - 1);   // an out-of-range draft is never accepted; its row is clamped
          }
          if (a.drafts && t + 1 == a.n_tokens && cs.w == 0 && tid_opaque() == 0 && a.out_accepted)
            gp(a.out_accepted)[0] = accepted;
        }
      }
      trace_flush(as, cs, st);
    }
  }
}
