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

template <int H_, int NH_, int QL_, int KL_, int RD_, int ND_, int VD_, int INTER_, bool FP8_, bool MOE_, bool SPARSE_>
struct MlaShape {
  static constexpr int H = H_, NH = NH_, QL = QL_, KL = KL_, RD = RD_, ND = ND_, VD = VD_, INTER = INTER_;
  static constexpr bool FP8 = FP8_, MOE = MOE_, SPARSE = SPARSE_;
  static constexpr int LAT = KL + RD, QH = ND + RD, ODIM = NH * VD;
  static constexpr int HPW = 8, NHG = NH / HPW;   // heads per attention workgroup, head groups
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

// ------------------------------------------------------------------ X: RMSNorm + [W_DQ ; W_DKV]
template <class SH>
__device__ __forceinline__ bool stage_x_mla(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const DLayer Ly = *gp(st.Ly);
  const int w = cx.w, nwg = cx.nwg;
  constexpr int R = SH::QL + SH::LAT;
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
    return layer_input<SH::H>(cx, a, st, L, gam, h0, h1);
  };
  seg_begin();
  int ns = 0;
  if (r0 < SH::QL) {
    seg_set(L, ns, Ly.w_dq.w + (size_t)r0 * RB, Ly.w_dq.s, min(r1, SH::QL) - r0, r0, 0, 1.f);
    ns++;
  }
  if (r1 > SH::QL) {
    const int lo = max(r0, SH::QL) - SH::QL;
    seg_set(L, ns, Ly.w_dkv.w + (size_t)lo * RB, Ly.w_dkv.s, r1 - max(r0, SH::QL), lo, 0, 1.f);
    ns++;
  }
  seg_end();
  if (!gemv_list<SH::FP8, SH::H, PLD_IF_QKV>(L.segs, ns, L.act, L.outb, OUT_STORE, pre_x)) return false;
  stamp(a, cx, st, TR_QKV_GEMV);
  if (!pre_x()) return false;
  __syncthreads();
  uint64_t* cqr = wsp<uint64_t>(a, a.off.cqr);
  uint64_t* ckvr = wsp<uint64_t>(a, a.off.ckvr);
  for (int r = r0 + tid_opaque(); r < r1; r += BLOCK) {
    const float v = L.outb[r - r0];
    if (r < SH::QL) ll_put_f32(cqr + r, v, st.k1);
    else ll_put_f32(ckvr + (r - SH::QL), v, st.k1);
  }
  stamp(a, cx, st, TR_QKV_DONE);
  return true;
}

// ------------------------------------------------------------------ Q: RMSNorm(c_q) + W_UQ + RoPE
template <class SH>
__device__ __forceinline__ bool stage_q_mla(Ctx& cx, const KArgs& a, const Step& st, Lds& L) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  const int w = cx.w, nwg = cx.nwg;
  constexpr int R = SH::NH * SH::QH;
  constexpr size_t RB = (size_t)SH::QL * (SH::FP8 ? 1 : 2);
  const int r0 = 2 * split_at(R / 2, nwg, w), r1 = 2 * split_at(R / 2, nwg, w + 1);
  RegVec<SH::QL> gq;
  gq.load(Ly.q_norm);
  bool pending = true;
  auto pre_q = [&]() -> bool {
    if (!pending) return true;
    pending = false;
    if (!ll_fetch<per_for(SH::QL)>(cx, reinterpret_cast<uint32_t*>(L.act), wsp<uint64_t>(a, a.off.cqr), SH::QL, st.k1,
                                   W_CQ))
      return false;
    rmsnorm_reg<SH::QL>(L.act, gq, c.eps, L.red);
    stamp(a, cx, st, TR_ATT_READY);
    return true;
  };
  seg_begin();
  seg_set(L, 0, Ly.w_uq.w + (size_t)r0 * RB, Ly.w_uq.s, r1 - r0, r0, 0, 1.f);
  seg_end();
  if (!gemv_list<SH::FP8, SH::QL, PLD_IF_WO>(L.segs, r1 > r0 ? 1 : 0, L.act, L.outb, OUT_STORE, pre_q)) return false;
  if (!pre_q()) return false;
  __syncthreads();
  const PLD_GLOBAL float* rope = gp(wsp<float>(a, a.off.rope)) + (size_t)st.pos * SH::RD;   // (cos, sin) pairs
  uint64_t* qn = wsp<uint64_t>(a, a.off.q);
  uint64_t* qr = wsp<uint64_t>(a, a.off.qr);
  for (int p = r0 / 2 + tid_opaque(); p < r1 / 2; p += BLOCK) {
    const int r = 2 * p, h = r / SH::QH, k = r % SH::QH;
    const float v0 = L.outb[r - r0], v1 = L.outb[r + 1 - r0];
    if (k < SH::ND) {
      ll_put_f32(qn + h * SH::ND + k, v0, st.k1);
      ll_put_f32(qn + h * SH::ND + k + 1, v1, st.k1);
    } else {
      const int d = k - SH::ND;
      const float cs = rope[d], sn = rope[d + 1];
      ll_put_f32(qr + h * SH::RD + d, v0 * cs - v1 * sn, st.k1);
      ll_put_f32(qr + h * SH::RD + d + 1, v0 * sn + v1 * cs, st.k1);
    }
  }
  stamp(a, cx, st, TR_ATT_Q);
  return true;
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
  float* red = L.act + SH::ND;          // [rpp][cpw]
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
  for (int e = 0; e < EPC; e++) red[rr * cpw + ck * EPC + e] = acc[e];
  __syncthreads();
  uint64_t* ql = wsp<uint64_t>(a, a.off.qlat) + (size_t)h * SH::KL + c0;
  for (int j = tid; j < cpw; j += BLOCK) {
    float s = 0.f;
    for (int g = 0; g < rpp; g++) s += red[g * cpw + j];
    ll_put_f32(ql + j, s, st.k1);
  }
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
  static_assert(KSTEPS % 4 == 0 && KL == 512 && HPW == NWAVES, "attention tiling");
  const int tid = tid_opaque();
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = c.cpg;
  const int hg = cx.w / nch, ch = cx.w % nch;
  const int hbase = hg * HPW;
  const int pos = st.pos, T = pos + 1;
  const int t0 = split_at(T, nch, ch), t1 = split_at(T, nch, ch + 1), n = t1 - t0;
  const int fresh = a.pos0;
  const int nst = max(0, min(n, fresh - t0));            // static rows of the chunk: [0, nst)
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
  auto srow = [&](int t) -> size_t { return (size_t)(nst > 0 ? t0 + min(t, nst - 1) : 0); };
  // Staging registers: three sub-blocks in flight (sets A, B, C in turn); chunk i of a
  // block covers (row i / CPRW, chunk i % CPRW). A block's loads are issued three blocks
  // before it is staged into LDS, so the wait at staging time covers ~3 blocks of work.
  // Rows are streamed through register sets A, B, C in turn: a block's loads are issued
  // DEPTH blocks before it is staged into LDS. All loads are unconditional (clamped rows;
  // blocks past the chunk read one uniform address and are masked), and a chunk that holds
  // rows written inside this launch reads all its rows coherently (the two load kinds are
  // separate template instances), so the in-order load waits stay exact. The row of
  // position pos is patched in from LDS after staging.
  constexpr int DEPTH = 3;
  const int nsb = (n + TB - 1) / TB;
  const int nsbp = (nsb + DEPTH - 1) / DEPTH * DEPTH;
  const bool coh = n > 0 && t0 + n > fresh;
  uint4 cb[DEPTH][NLD];
  auto issue = [&](int set, int sb, auto coh_tag) {
    constexpr bool COH = decltype(coh_tag)::value;
    const bool live = sb < nsb;
#pragma unroll
    for (int i = 0; i < NLD; i++) {
      const int idx = min(tid + i * BLOCK, TB * CPRW - 1);
      const int r = idx / CPRW, k = idx % CPRW;
      const int t = max(min(sb * TB + r, n - 1), 0);
      const size_t row = COH ? (size_t)(t0 + t) : srow(t);
      const uint16_t* p = live ? lat + row * LAT + k * 8 : lat;
      cb[set][i] = COH ? ld_coh16(p) : ld_g16(p);
    }
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
    const int rp = pos - t0 - sb * TB;   // row of pos inside this block
    if (rp >= 0 && rp < TB && pos < t1) {
      __syncthreads();
      for (int k = tid; k < LAT / 2; k += BLOCK)
        reinterpret_cast<uint32_t*>(C + rp * CSTR)[k] = reinterpret_cast<const uint32_t*>(newrow)[k];
    }
  };
  if (coh) {
#pragma unroll
    for (int d = 0; d < DEPTH; d++) issue(d, d, std::true_type{});
  } else {
#pragma unroll
    for (int d = 0; d < DEPTH; d++) issue(d, d, std::false_type{});
  }
  // q of the head group: q_lat [HPW][KL] and q_rope [HPW][RD] (LL) -> bf16 rows of Qs
  if (!ll_fetch<per_for(HPW * KL)>(cx, reinterpret_cast<uint32_t*>(qtmp),
                                   wsp<uint64_t>(a, a.off.qlat) + (size_t)hbase * KL, HPW * KL, k1, W_QLAT))
    return false;
  if (!ll_fetch<per_for(HPW * RD)>(cx, reinterpret_cast<uint32_t*>(qtmp + HPW * KL),
                                   wsp<uint64_t>(a, a.off.qr) + (size_t)hbase * RD, HPW * RD, k1, W_QLAT))
    return false;
  for (int i = tid; i < 16 * LAT; i += BLOCK) {
    const int h = i / LAT, k = i % LAT;
    const float v = h >= HPW ? 0.f : (k < KL ? qtmp[h * KL + k] : qtmp[HPW * KL + h * RD + (k - KL)]);
    Qs[h * CSTR + k] = (uint16_t)bf16_bits(v);
  }
  for (int i = tid; i < 16 * TB; i += BLOCK) Ps[i] = 0;
  // the row of position pos (chunk that holds it): RMSNorm(c_kv') and RoPE(k_r'), bf16
  if (t0 <= pos && pos < t1) {
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
      float v0, v1;
      if (k < KL) {
        v0 = (float)(((double)ntmp[k] * r) * (double)g[k]);
        v1 = (float)(((double)ntmp[k + 1] * r) * (double)g[k + 1]);
      } else {
        const int d = k - KL;
        const float x0 = ntmp[k], x1 = ntmp[k + 1], cs = rope[d], sn = rope[d + 1];
        v0 = x0 * cs - x1 * sn;
        v1 = x0 * sn + x1 * cs;
      }
      const uint32_t pair = f32_to_bf16(v0) | (f32_to_bf16(v1) << 16);
      reinterpret_cast<uint32_t*>(newrow)[i] = pair;
      if (hg == 0) st_u32(reinterpret_cast<uint32_t*>(Ly.lat + (size_t)pos * LAT) + i, pair);   // cache append
    }
  }
  __syncthreads();
  stamp(a, cx, st, TR_ATT_READY);
  const float scale = 1.0f / sqrtf((float)(SH::ND + SH::RD));
  float m_run = -INFINITY, l_run = 0.f;   // wave h < HPW: head h
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
    // ---- online softmax: wave h owns head h; lane t < TB is token tb0 + t
    {
      const int h = wave;
      float s = -INFINITY;
      if (lane < TB && tb0 + lane < n) {
        const int nt = lane >> 4, col = lane & 15;
        s = 0.f;
#pragma unroll
        for (int kq = 0; kq < 4; kq++) s += Ssc[(kq * 2 + nt) * 256 + h * 16 + col];
        s *= scale;
      }
      const float mb = wave_max_dpp(s);
      const float mnew = fmaxf(m_run, mb);
      const float al = m_run == -INFINITY ? 0.f : __expf(m_run - mnew);
      const float p = s == -INFINITY ? 0.f : __expf(s - mnew);
      l_run = l_run * al + wave_sum_dpp(p);
      m_run = mnew;
      if (lane < TB) Ps[h * TB + lane] = (uint16_t)bf16_bits(p);
      if (lane == 0) alph[h] = al;
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
  auto main_loop = [&](auto coh_tag) {
    for (int sb0 = 0; sb0 < nsbp; sb0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; d++) {
        const int sb = sb0 + d;
        const int tb0 = sb * TB, buf = sb & 1;
        const uint16_t* C = Cs + buf * TB * CSTR;
        store(d, sb, buf);
        __syncthreads();
        if (sb == 0) stamp(a, cx, st, 17);
        issue(d, sb + DEPTH, coh_tag);   // refill this set, DEPTH blocks ahead
        block(C, tb0);
        if (sb == 0) stamp(a, cx, st, 31);
      }
    }
  };
  if (coh) main_loop(std::true_type{});
  else main_loop(std::false_type{});
  stamp(a, cx, st, TR_ATT_SOFTMAX);
  // publish the partial of each head: LL words [m, l, acc[0..KL)] at ((h * nch) + ch) * (KL + 2)
  vm_wait();   // the cache row appended above is visible before this workgroup's next publication
  __syncthreads();
  uint64_t* pll = wsp<uint64_t>(a, a.off.part);
  if (lane == 0 && wave < HPW) {
    uint64_t* p = pll + ((size_t)(hbase + wave) * nch + ch) * (KL + 2);
    ll_put_f32(p, m_run, k1);
    ll_put_f32(p + 1, l_run, k1);
  }
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const int col = (wave * 4 + t) * 16 + ln;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int h = 4 * lq + q;
      if (h < HPW) ll_put_f32(pll + ((size_t)(hbase + h) * nch + ch) * (KL + 2) + 2 + col, O[t][q], k1);
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
  const int nacc = nch * cpw;
  auto pidx = [=](int i) -> int {
    if (i < nacc) return (h * nch + i / cpw) * (KL + 2) + 2 + c0 + i % cpw;
    const int j = i - nacc;
    return (h * nch + (j >> 1)) * (KL + 2) + (j & 1);
  };
  float* accs = L.act;              // [nch][cpw]
  float* mls = L.act + nacc;        // [nch][2]
  float* fw = mls + 2 * nch;        // [nch]
  float* lsum = fw + nch;           // [1]
  stamp(a, cx, st, TR_MERGE_START);
  if (!ll_fetch<per_for(4096 + 64)>(cx, reinterpret_cast<uint32_t*>(L.act), wsp<uint64_t>(a, a.off.part),
                                    nacc + 2 * nch, st.k1, W_PART, pidx))
    return false;
  stamp(a, cx, st, TR_MERGE_COPIED);
  if (wave == 0) {
    float M = -INFINITY;
    for (int cc = lane; cc < nch; cc += 64)
      if (mls[2 * cc + 1] > 0.f) M = fmaxf(M, mls[2 * cc]);
    M = wave_max(M);
    float ls = 0.f;
    for (int cc = lane; cc < nch; cc += 64) {
      const float l = mls[2 * cc + 1];
      const float f = l > 0.f ? __expf(mls[2 * cc] - M) : 0.f;
      fw[cc] = f;
      ls += f * l;
    }
    ls = wave_sum(ls);
    if (lane == 0) lsum[0] = ls;
  }
  __syncthreads();
  uint64_t* ol = wsp<uint64_t>(a, a.off.olat) + (size_t)h * KL + c0;
  for (int j = tid; j < cpw; j += BLOCK) {
    float o = 0.f;
#pragma unroll 8
    for (int cc = 0; cc < nch; cc++) o = fmaf(fw[cc], accs[cc * cpw + j], o);
    ll_put_f32(ol + j, o / lsum[0], st.k1);
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
                                   wsp<uint64_t>(a, a.off.olat) + (size_t)h * SH::KL, SH::KL, st.k1, W_OLAT))
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
  const DLayer* layers = wsp<DLayer>(a, a.off.layers);
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
      KArgs as = a;
      asm volatile("" : "+s"(as.ws));
      uint32_t lds0 = 0;
      asm volatile("" : "+s"(lds0));
      Lds L = carve(lds_raw + lds0, a.c);
      st.tr = L.tr;
      stamp(as, cx, st, TR_START);
      if (!stage_x_mla<SH>(cx, as, st, L)) return;
      if (!stage_q_mla<SH>(cx, as, st, L)) return;
      if (!stage_absorb_mla<SH>(cx, as, st, L)) return;
      if (!stage_attn_mla<SH>(cx, as, st, L)) return;
      if (!stage_merge_mla<SH>(cx, as, st, L)) return;
      if (!stage_uv_mla<SH>(cx, as, st, L)) return;
      if (!stage_wo<SH>(cx, as, st, L)) return;
      if (!stage_ffn<SH>(cx, as, st, L)) return;
      if (!stage_down<SH>(cx, as, st, L, last ? as.out_hidden : nullptr)) return;
      if constexpr (SH::FP8) {
        if (a.head_on && li == a.n_layers - 1 && !stage_head<SH>(cx, as, st, L, t, &token)) return;
      }
      trace_flush(as, cx, st);
    }
  }
}
