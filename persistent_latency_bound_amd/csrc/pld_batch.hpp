// Batched verify of the FP8 MLA stack: the nq positions of one multi-token verify go
// through every layer TOGETHER, so each weight is read from HBM once per step instead of
// once per position (included by pld_kernel.hip after pld_mla.hpp).
//
// The vLLM Kimi K3 backend article scores the speculative drafts of one request in one
// forward pass (summary and "Throughput holds across the tested range": DSpark with an
// acceptance length of six), and names shape-aware matmuls as one of its four changes
// ("Four changes drive the gains"). With nq <= 8 positions each dense projection is a
// skinny GEMM [rows x K] x [K x nq]: on gfx950 it runs on the matrix cores,
// v_mfma_f32_16x16x32_bf16, with the FP8 weights converted to bf16 in registers (exact:
// every E4M3 value is a bf16 value) and their fp32 block scale applied to each 64-wide
// k-step's fp32 partial. The activations enter the matrix cores as bf16 (one rounding of
// each normalised input); accumulation is fp32.
//
// One batched step of a layer (LL buffers hold nq copies, one per position):
//   BX  a_p = RMSNorm(x_p); [c_q' ; c_kv' | k_r']_p = [W_DQ ; W_DKV] a_p      (matrix cores)
//   BQ  RMSNorm(c_q'_p); q_p = W_UQ c_q_p, RoPE at position pos + p          (matrix cores)
//   BA  q_lat = W_UK^T q_nope per head and position (weights in registers, reused)
//   BT  attention. Verify: per (8-head group, chunk of the shared history), all positions
//       in one pass over the chunk; the nq new latent rows join the last chunk with the
//       causal mask (position p sees new rows 0..p). Batch decode: per (16-head group,
//       sequence, chunk of that sequence's history), one pass; the sequence's new row
//       joins its last chunk
//   BM  merge of the chunk partials, per position
//   BU  o = W_UV o_lat per head                                               (matrix cores)
//   BO  h2_p = x_p + W_O o_p                                                  (matrix cores)
//       and, over this workgroup's rows, the partial sums that BF needs
//   BF  RMSNorm(h2_p) and the router logits in fp64 (the selection must match an fp64
//       evaluation), both from partial sums that the W_O workgroups form over their own
//       rows (sum of h2^2; sum of W_r * gamma * h2 per expert): the router no longer waits
//       for the whole h2; shared experts (matrix cores); the top-k of every position at
//       once; the UNION of the selected experts, each read once for the positions that
//       chose it (matrix cores)
//   BD  down projections: this workgroup's output rows for every (expert, position)
//       pair, the expert's rows read once; f_p = sum of gated results; x'_p = h2_p + f_p
// then, after the last layer, the LM head and the token choice of each position and the
// acceptance count.
#pragma once

constexpr int VB = 8;                    // positions per batched step (max)
constexpr int VACT_BYTES = 150528;       // LDS region for matrix-core operands / attention (147 KiB)

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ matrix-core segment list
// A segment is n consecutive FP8 rows of one matrix (row stride K bytes, block scales s
// with scale row (srow + r) >> 7). Its A operand: position p reads the bf16 vector at
// A + a_off + vrow[p] * (K + 8) (LDS), or zeros when vrow[p] < 0. Results: position p,
// row r at out[o_off + p * ostr + r].
struct MSeg {
  const uint8_t* w;
  const float* s;
  int n, srow, a_off, o_off;
  int8_t vrow[VB];
};
constexpr int MAX_MSEGS = 24;
__device__ __forceinline__ constexpr int vb_astr(int K) { return K + 8; }   // bf16 elements per A row

__device__ __forceinline__ void mseg_set(MSeg* segs, int i, const uint8_t* w, const float* s, int n, int srow,
                                         int a_off, int o_off, int nq) {
  if (tid_opaque() == 0) {
    MSeg& S = segs[i];
    S.w = w; S.s = s; S.n = n; S.srow = srow; S.a_off = a_off; S.o_off = o_off;
    for (int p = 0; p < VB; p++) S.vrow[p] = (int8_t)(p < nq ? p : -1);
  }
}

// Rows of a segment list times up to 16 activation rows on the matrix cores.
//  * Each segment is cut into tiles of 16 rows (the last one partial: its spare columns
//    reload the segment's last row, which costs no extra HBM bytes); tile t is the B
//    operand of v_mfma_f32_16x16x32_bf16, lane (n, g) = (lane & 15, lane >> 4) holding row n.
//  * An item is a 128-wide k-step of a tile: two 16-byte loads per lane, each covering 8
//    rows x 128 contiguous bytes (whole cache lines): the first, rows 0..7, lane (n, g)
//    reading row n & 7 at byte 64 (n >> 3) + 16 g; the second the same for rows 8..15. A
//    rotate by 8 lanes inside each 16-lane row (DPP) then leaves lane (n, g) with row n's
//    bytes [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g + 16): four products of 32 k (the k
//    order inside a product is the same permutation on both operands). Loading 16 rows x
//    64 bytes per instruction instead (the plain layout) ran the stream ~12% slower.
//  * Work units are (tile, k-slice): with fewer than 8 tiles, K is split into KS slices
//    so that every wave of the workgroup streams; the slices' partial sums are added in
//    slice order afterwards (fixed order, so results do not depend on timing).
//  * Each wave streams its units as one pipeline with D items (2 D loads) in flight per
//    lane; the first D are issued before pre() (the dependency wait), like the vector GEMV.
//  * The fp32 block scale of the lane's row multiplies each item's partial product (the
//    output column of a lane is its own B row, so the lane holds its own scale; an item
//    lies in one 128-wide scale block).
// `segs` lives in LDS; `part` is LDS scratch of 8 * 16 * VB floats; ostr 0 means each
// segment's own row count. Returns false if pre() reported an abort. Ends with a
// workgroup barrier.
__device__ __forceinline__ uint4 ror8_rows(uint4 v) {
  uint4 r;
  r.x = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.x, 0x128, 0xf, 0xf, false);   // row_ror:8
  r.y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.y, 0x128, 0xf, 0xf, false);
  r.z = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.z, 0x128, 0xf, 0xf, false);
  r.w = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.w, 0x128, 0xf, 0xf, false);
  return r;
}
__device__ __forceinline__ void fp8x16_to_bf16(const uint4& v, bf16x8_t& b0, bf16x8_t& b1) {
  const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
  uint32_t bw[8];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const bf16x2_v lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[i], 1.0f, false);
    const bf16x2_v hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[i], 1.0f, true);
    bw[2 * i] = __builtin_bit_cast(uint32_t, lo);
    bw[2 * i + 1] = __builtin_bit_cast(uint32_t, hi);
  }
  b0 = __builtin_bit_cast(bf16x8_t, make_uint4(bw[0], bw[1], bw[2], bw[3]));
  b1 = __builtin_bit_cast(bf16x8_t, make_uint4(bw[4], bw[5], bw[6], bw[7]));
}

template <int K, int D, typename Pre>
__device__ __forceinline__ bool mfma_list(const MSeg* segs, int nseg, const uint16_t* A, float* out, int ostr,
                                          float* part, int nq, Pre&& pre) {
  static_assert(K % 128 == 0, "whole 128-wide items");
  constexpr int AST = vb_astr(K);
  constexpr int SBK = (K + 127) / 128;
  const int tid = tid_opaque(), lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const bool lo8 = n < 8;
  int ntiles = 0;
  for (int s = 0; s < nseg; s++) ntiles += (segs[s].n + 15) >> 4;
  int KS = 1;
  if (ntiles > 0 && ntiles < NWAVES) {
    KS = NWAVES / ntiles;
    while ((K / 128) % KS) KS--;
  }
  const int NS = K / 128 / KS;                  // items per unit
  const int nunits = ntiles * KS;
  const int myunits = wave < nunits ? (nunits - wave + NWAVES - 1) / NWAVES : 0;
  const int nit = myunits * NS;
  // The item loop below runs in whole groups of D with unconditional loads: a load issued
  // under a condition leaves the compiler unsure how many are in flight, and it then waits
  // for all of them before every use (the stream would run one load deep). Past the last
  // item, loads repeat the last address and results are discarded.
  const int nitD = (nit + D - 1) / D * D;
  // unit -> (segment, tile in segment, slice)
  auto unit_of = [&](int ui, int* sg, int* tt, int* q) {
    const int u = wave + ui * NWAVES;
    int t = u % ntiles;
    *q = u / ntiles;
    int s = 0;
    for (; s < nseg - 1; s++) {
      const int nt = (segs[s].n + 15) >> 4;
      if (t < nt) break;
      t -= nt;
    }
    *sg = s;
    *tt = t;
  };
  // issue cursor: unit iu, item is; per-unit row pointers of the lane's two loads
  int iu = 0, is = 0;
  const uint8_t* wa = nullptr;   // row (n & 7) of the tile, at this lane's byte offset
  const uint8_t* wb = nullptr;   // row 8 + (n & 7)
  const PLD_GLOBAL float* srow = nullptr;
  int kbeg = 0;
  auto open_unit = [&](int ui) {
    int sg, tt, q;
    unit_of(ui, &sg, &tt, &q);
    const MSeg& S = segs[sg];
    const int ra = min(16 * tt + (n & 7), S.n - 1), rb = min(16 * tt + 8 + (n & 7), S.n - 1);
    const int rn = min(16 * tt + n, S.n - 1);
    kbeg = q * (K / KS);
    wa = S.w + (size_t)ra * K + kbeg + 64 * (n >> 3) + 16 * g;
    wb = S.w + (size_t)rb * K + kbeg + 64 * (n >> 3) + 16 * g;
    srow = gp(S.s) + (size_t)((S.srow + rn) >> 7) * SBK + (kbeg >> 7);
  };
  uint4 bufa[D], bufb[D];
  float scb[D];
  auto issue = [&](int d) {
    bufa[d] = ld_stream16(wa + 128 * is);
    bufb[d] = ld_stream16(wb + 128 * is);
    scb[d] = srow[is];
    if (is + 1 < NS) {
      is++;
    } else if (iu + 1 < myunits) {
      is = 0;
      iu++;
      open_unit(iu);
    }
  };
  if (myunits > 0) {
    open_unit(0);
#pragma unroll
    for (int d = 0; d < D; d++) issue(d);
  }
  if (!pre()) return false;
  // compute cursor
  int cu = 0, cs = 0;
  const uint16_t* arow = nullptr;
  int csg = 0, ctt = 0, cq = 0;
  auto open_compute = [&](int ui) {
    unit_of(ui, &csg, &ctt, &cq);
    const MSeg& S = segs[csg];
    const int vr = (n < VB) ? (int)S.vrow[n] : -1;
    arow = vr >= 0 ? A + S.a_off + vr * AST + cq * (K / KS) + 16 * g : nullptr;
  };
  if (myunits > 0) open_compute(0);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int it0 = 0; it0 < nitD; it0 += D) {
#pragma unroll
    for (int d = 0; d < D; d++) {
      const bool live = it0 + d < nit;
      uint4 a0 = make_uint4(0u, 0u, 0u, 0u), a1 = a0, a2 = a0, a3 = a0;
      if (arow) {
        const uint16_t* ap = arow + 128 * cs;
        a0 = *reinterpret_cast<const uint4*>(ap);
        a1 = *reinterpret_cast<const uint4*>(ap + 8);
        a2 = *reinterpret_cast<const uint4*>(ap + 64);
        a3 = *reinterpret_cast<const uint4*>(ap + 72);
      }
      const uint4 va = bufa[d], vb = bufb[d];
      const float sc = scb[d];
      issue(d);
      const uint4 ra = ror8_rows(va), rb = ror8_rows(vb);
      const uint4 p0 = lo8 ? va : rb, p1 = lo8 ? ra : vb;   // row n: bytes [16 g, +16) and [64 + 16 g, +16)
      bf16x8_t b0, b1, b2, b3;
      fp8x16_to_bf16(p0, b0, b1);
      fp8x16_to_bf16(p1, b2, b3);
      f32x4_t pk = {0.f, 0.f, 0.f, 0.f};
      pk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0), b0, pk, 0, 0, 0);
      pk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1), b1, pk, 0, 0, 0);
      pk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a2), b2, pk, 0, 0, 0);
      pk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a3), b3, pk, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; i++) acc[i] = fmaf(sc, pk[i], acc[i]);
      if (live && ++cs == NS) {
        // unit done: lane holds rows p = 4 g + i of column n
        const MSeg& S = segs[csg];
        const int r = 16 * ctt + n;
        if (r < S.n) {
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int p = 4 * g + i;
            if (p < nq) {
              if (KS == 1) out[S.o_off + p * (ostr ? ostr : S.n) + r] = acc[i];
              else part[((cq * ntiles + (wave + cu * NWAVES) % ntiles) * 16 + n) * VB + p] = acc[i];
            }
          }
        }
        acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        cs = 0;
        if (++cu < myunits) open_compute(cu);
      }
    }
  }
  __syncthreads();
  if (KS > 1) {
    // slice partials of tile t, column n, position p, added in slice order
    for (int i = tid; i < ntiles * 16 * VB; i += BLOCK) {
      const int p = i % VB, nn = (i / VB) % 16, t = i / (16 * VB);
      if (p >= nq) continue;
      int s = 0, tt = t;
      for (; s < nseg - 1; s++) {
        const int nt = (segs[s].n + 15) >> 4;
        if (tt < nt) break;
        tt -= nt;
      }
      const int r = 16 * tt + nn;
      if (r >= segs[s].n) continue;
      float v = 0.f;
      for (int q = 0; q < KS; q++) v += part[((q * ntiles + t) * 16 + nn) * VB + p];
      out[segs[s].o_off + p * (ostr ? ostr : segs[s].n) + r] = v;
    }
    __syncthreads();
  }
  return true;
}

// ------------------------------------------------------------------ LDS of the batched kernel
struct VLds {
  uint16_t* A;     // [VACT_BYTES] matrix-core A rows / attention / merge scratch (also used as floats)
  float* out;      // [VB * 64]     stage results (rows of this workgroup x positions)
  float* part;     // [8 * 16 * VB] k-slice partials
  float* xres;     // [VB][32]      this workgroup's rows of each position's layer input
  float* h2res;    // [VB][32]      ... and of h2
  int* vslot;      // [VB][8] (+ pad to VB * 32 ints) union slot of each position's top-k expert
  double* red;     // [16]
  double* redv;    // [NWAVES][VB]  per-position block reductions
  int* isel;       // [VB][8]       per-position top-k experts (rank order)
  float* fgate;    // [VB][8]       their gates
  int* uexp;       // [VB * 8 + 4]  union of the selected experts (ascending), then shared
  int* umask;      // [VB * 8 + 4]  positions that use each union slot (bit p)
  int* misc;       // [16]          union size; misc + 8: the head stage's argmax slot
  int* tok;        // [2 * VB]      input tokens of the rows, then the chosen tokens
  int* rpos;       // [VB]          cache position of each row in the current step
  int* pcs;        // [3 * MAX_MSEGS / 2] routed pieces of this workgroup: union slot, j0, j1
  int* vsrc;       // [32]          down pass: LL word offset of each fetched (slot, position) vector
  MSeg* segs;      // [MAX_MSEGS]
  uint64_t* tr;    // [TR_SLOTS]
  double* dk;      // [16]
  double* vnorm;   // [VB]          FFN norm scale of each position (W_O stage -> FFN stage)
  uint32_t* stage; // [3 * 1024]    LL staging for the head's inputs (aliases nothing live)
};
constexpr int VOUT_FLOATS = VB * 64;
__host__ __device__ inline size_t vlds_bytes() {
  return (size_t)VACT_BYTES + 4 * (VOUT_FLOATS + 8 * 16 * VB + 3 * VB * 32) + 8 * 16 + 8 * NWAVES * VB + 4 * (VB * 8) * 2 +
         4 * 2 * (VB * 8 + 4) + 4 * 16 + 4 * 2 * VB + 4 * VB + 4 * 3 * (MAX_MSEGS / 2) + 4 * 32 + sizeof(MSeg) * MAX_MSEGS +
         8 * TR_SLOTS + 8 * 16 + 8 * VB;
}
__device__ __forceinline__ VLds vcarve(float* base) {
  VLds L;
  char* p = reinterpret_cast<char*>(base);
  L.A = reinterpret_cast<uint16_t*>(p); p += VACT_BYTES;
  L.out = reinterpret_cast<float*>(p); p += 4 * VOUT_FLOATS;
  L.part = reinterpret_cast<float*>(p); p += 4 * 8 * 16 * VB;
  L.xres = reinterpret_cast<float*>(p); p += 4 * VB * 32;
  L.h2res = reinterpret_cast<float*>(p); p += 4 * VB * 32;
  L.vslot = reinterpret_cast<int*>(p); p += 4 * VB * 32;
  L.red = reinterpret_cast<double*>(p); p += 8 * 16;
  L.redv = reinterpret_cast<double*>(p); p += 8 * NWAVES * VB;
  L.isel = reinterpret_cast<int*>(p); p += 4 * VB * 8;
  L.fgate = reinterpret_cast<float*>(p); p += 4 * VB * 8;
  L.uexp = reinterpret_cast<int*>(p); p += 4 * (VB * 8 + 4);
  L.umask = reinterpret_cast<int*>(p); p += 4 * (VB * 8 + 4);
  L.misc = reinterpret_cast<int*>(p); p += 4 * 16;
  L.tok = reinterpret_cast<int*>(p); p += 4 * 2 * VB;
  L.rpos = reinterpret_cast<int*>(p); p += 4 * VB;
  L.pcs = reinterpret_cast<int*>(p); p += 4 * 3 * (MAX_MSEGS / 2);
  L.vsrc = reinterpret_cast<int*>(p); p += 4 * 32;
  L.segs = reinterpret_cast<MSeg*>(p); p += sizeof(MSeg) * MAX_MSEGS;
  L.tr = reinterpret_cast<uint64_t*>(p); p += 8 * TR_SLOTS;
  L.dk = reinterpret_cast<double*>(p); p += 8 * 16;
  L.vnorm = reinterpret_cast<double*>(p);
  L.stage = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(base) + 98432);   // inside A, past 8 rows of K = 6144
  return L;
}

// The head stage of the single-position path runs once per position on this LDS: its
// activation and candidate areas map into the A region.
__device__ __forceinline__ Lds head_lds(const VLds& V) {
  Lds L;
  L.act = reinterpret_cast<float*>(V.A);                                       // [H] doubles = 48 KiB
  L.stage = V.stage;                                                           // [H/2] words
  L.outb = reinterpret_cast<float*>(reinterpret_cast<char*>(V.A) + 122880);    // [vocab/nwg] doubles
  L.outc = nullptr;
  L.xres = L.h2res = nullptr;
  L.red = V.red;
  L.isel = V.misc + 8;
  L.fgate = nullptr;
  L.segs = nullptr;
  L.tr = V.tr;
  L.dk = V.dk;
  L.pcs = nullptr;
  return L;
}

// Per-position LL buffers: buffer b of position p.
template <typename T = uint64_t>
__device__ __forceinline__ uint64_t* vbuf(const KArgs& a, size_t off, size_t words, int p) {
  return wsp<uint64_t>(a, off) + (size_t)p * words;
}

// LL fetch of nq per-position vectors of N words: position p's words at src + p * sstride
// (LL words), into dst + p * dstride (32-bit words, LDS); one pass, all loads in flight.
template <int N>
struct IdxRows {
  int sstride;
  __device__ __forceinline__ int operator()(int i) const { return (i / N) * sstride + i % N; }
};
template <int N>
struct StRows {
  int dstride;
  __device__ __forceinline__ void operator()(uint32_t* dst, int i, uint32_t v) const { dst[(i / N) * dstride + i % N] = v; }
};
// (up to 24 loads per thread and round: each round is a full round trip, and the per-position
// handoffs of up to 8 rows are several times larger than the single-position ones)
constexpr int per_rows(int n) { return (n + BLOCK - 1) / BLOCK > 24 ? 24 : (n + BLOCK - 1) / BLOCK; }
template <int N>
__device__ __forceinline__ bool ll_fetch_rows(Ctx& cx, uint32_t* dst, int dstride, const uint64_t* src, int sstride,
                                              int nq, uint32_t ep, int wid) {
  return ll_fetch<per_rows(VB * N)>(cx, dst, src, nq * N, ep, wid, IdxRows<N>{sstride}, StRows<N>{dstride});
}

// Sums over the workgroup of VB per-thread values at once (one pair of barriers); every
// thread gets the totals.
__device__ __forceinline__ void block_sum_rows(double (&v)[VB], double* redv) {
  const int lane = tid_opaque() & 63, wave = tid_opaque() >> 6;
#pragma unroll
  for (int p = 0; p < VB; p++) v[p] = wave_sum_any(v[p]);
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int p = 0; p < VB; p++) redv[wave * VB + p] = v[p];
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < VB; p++) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < NWAVES; w++) t += redv[w * VB + p];
    v[p] = t;
  }
  __syncthreads();
}

// Element pairs (2j, 2j + 1), j = tid + k * BLOCK, of a length-N fp32 vector in registers
// (norm gains, loaded before a stage's weight stream is issued).
template <int N>
struct RegPairs {
  static constexpr int K = (N / 2 + BLOCK - 1) / BLOCK;
  float2 v[K];
  __device__ __forceinline__ void load(const float* p) {
    const PLD_GLOBAL float2* g = gp(reinterpret_cast<const float2*>(p));
#pragma unroll
    for (int k = 0; k < K; k++) {
      const int j = tid_opaque() + k * BLOCK;
      v[k] = make_float2(0.f, 0.f);
      if ((N / 2) % BLOCK == 0 || j < N / 2) {
        const float2 t = g[j];
        v[k] = t;
      }
    }
  }
};

// Sums over the workgroup of VB per-thread fp32 values at once (one pair of barriers).
__device__ __forceinline__ void block_sum_rows_f32(float (&v)[VB], double* redv) {
  float* red = reinterpret_cast<float*>(redv);   // [NWAVES][VB]
  const int lane = tid_opaque() & 63, wave = tid_opaque() >> 6;
#pragma unroll
  for (int p = 0; p < VB; p++) v[p] = wave_sum_dpp(v[p]);
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int p = 0; p < VB; p++) red[wave * VB + p] = v[p];
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < VB; p++) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVES; w++) t += red[w * VB + p];
    v[p] = t;
  }
  __syncthreads();
}

// RMSNorm of the nq rows of an N-vector into the bf16 A rows A + p * astr (the matrix cores
// take bf16 operands, whose rounding, 2^-9, is far above that of fp32 statistics, so the
// statistics and the product are fp32 here): y = (x * r) * gamma, r = 1/sqrt(sum(x^2)/N + eps).
// The input pair (p, j) is ld(p, j) (elements 2j, 2j + 1; LDS; it may be the A row itself:
// each pair is read and then written by the same thread); the fp32 y also to f32 + p * fstr
// when f32 is set. A thread's pairs of one row are read together before any write.
template <int N, typename Ld>
__device__ __forceinline__ void rms_rows(uint16_t* A, int astr, Ld&& ld, const RegPairs<N>& gam, double eps,
                                         double* redv, int nq, float* f32 = nullptr, int fstr = 0) {
  constexpr int KK = RegPairs<N>::K;
  static_assert(N % 2 == 0, "pairs");
  float ss[VB];
#pragma unroll
  for (int p = 0; p < VB; p++) {
    ss[p] = 0.f;
    if (p < nq) {
      float2 xv[KK];
#pragma unroll
      for (int k = 0; k < KK; k++) {
        const int j = tid_opaque() + k * BLOCK;
        xv[k] = ((N / 2) % BLOCK == 0 || j < N / 2) ? ld(p, j) : make_float2(0.f, 0.f);
      }
#pragma unroll
      for (int k = 0; k < KK; k++) ss[p] = fmaf(xv[k].x, xv[k].x, fmaf(xv[k].y, xv[k].y, ss[p]));
    }
  }
  block_sum_rows_f32(ss, redv);
#pragma unroll
  for (int p = 0; p < VB; p++) {
    if (p < nq) {
      const float r = 1.0f / sqrtf(ss[p] / (float)N + (float)eps);
      float2 xv[KK];
#pragma unroll
      for (int k = 0; k < KK; k++) {
        const int j = tid_opaque() + k * BLOCK;
        xv[k] = ((N / 2) % BLOCK == 0 || j < N / 2) ? ld(p, j) : make_float2(0.f, 0.f);
      }
#pragma unroll
      for (int k = 0; k < KK; k++) {
        const int j = tid_opaque() + k * BLOCK;
        if ((N / 2) % BLOCK == 0 || j < N / 2) {
          const float y0 = (xv[k].x * r) * gam.v[k].x, y1 = (xv[k].y * r) * gam.v[k].y;
          reinterpret_cast<uint32_t*>(A + p * astr)[j] = f32_to_bf16(y0) | (f32_to_bf16(y1) << 16);
          if (f32) reinterpret_cast<float2*>(f32 + p * fstr)[j] = make_float2(y0, y1);
        }
      }
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------ BX
template <class SH>
__device__ __forceinline__ bool bstage_x(Ctx& cx, const KArgs& a, const Step& st, VLds& L, int nq, int li) {
  const DLayer Ly = *gp(st.Ly);
  const int w = cx.w, nwg = cx.nwg;
  constexpr int H = SH::H, R = SH::QL + SH::LAT, AST = vb_astr(H);
  // W_DQ rows over the first nwq workgroups, W_DKV rows over the rest (in proportion), so
  // that no workgroup holds rows of both (two segments: two 16-row tiles and twice the items
  // per wave for the one workgroup that did)
  const int nwq = max(1, min(nwg - 1, (int)(((long long)nwg * SH::QL + R / 2) / R)));
  const int r0 = w < nwq ? split_at(SH::QL, nwq, w) : SH::QL + split_at(SH::LAT, nwg - nwq, w - nwq);
  const int r1 = w < nwq ? split_at(SH::QL, nwq, w + 1) : SH::QL + split_at(SH::LAT, nwg - nwq, w - nwq + 1);
  int h0, h1;
  hrows(H, nwg, w, &h0, &h1);
  RegPairs<H> gam;
  gam.load(Ly.attn_norm);
  {
    __syncthreads();
    int ns = 0;
    if (r0 < SH::QL) {
      mseg_set(L.segs, ns, Ly.w_dq.w + (size_t)r0 * H, Ly.w_dq.s, min(r1, SH::QL) - r0, r0, 0, 0, nq);
      ns++;
    }
    if (r1 > SH::QL) {
      const int lo = max(r0, SH::QL) - SH::QL;
      mseg_set(L.segs, ns, Ly.w_dkv.w + (size_t)lo * H, Ly.w_dkv.s, r1 - max(r0, SH::QL), lo, 0,
               max(r0, SH::QL) - r0, nq);
      ns++;
    }
    __syncthreads();
    auto pre = [&]() -> bool {
      // the nq inputs as bf16 rows in place: embedding rows (first layer) or the previous
      // layer's outputs (LL words of bf16 pairs), all fetched together
      if (li == 0) {
        for (int p = 0; p < nq; p++) {
          const PLD_GLOBAL uint32_t* src = gp(reinterpret_cast<const uint32_t*>(a.embed + (size_t)L.tok[p] * H));
          uint32_t* Aw = reinterpret_cast<uint32_t*>(L.A + p * AST);
          for (int i = tid_opaque(); i < H / 2; i += BLOCK) Aw[i] = src[i];
        }
        __syncthreads();
      } else if (!ll_fetch_rows<H / 2>(cx, reinterpret_cast<uint32_t*>(L.A), AST / 2, vbuf(a, a.off.vx, H / 2, 0), H / 2,
                                       nq, st.k1 - 1u, W_X)) {
        return false;
      }
      stamp(a, cx, st, TR_X_READY);
      for (int i = tid_opaque(); i < nq * (h1 - h0); i += BLOCK) {
        const int p = i / (h1 - h0), r = h0 + i % (h1 - h0);
        L.xres[p * 32 + (r - h0)] = bf16_to_f32(L.A[p * AST + r]);
      }
      __syncthreads();
      rms_rows<H>(L.A, AST, [&](int p, int j) {
        const uint32_t v = reinterpret_cast<const uint32_t*>(L.A + p * AST)[j];
        return make_float2(bf_lo(v), bf_hi(v));
      }, gam, a.c.eps, L.redv, nq);
      stamp(a, cx, st, TR_X_NORMED);
      return true;
    };
    if (!mfma_list<H, 4>(L.segs, ns, L.A, L.out, r1 - r0, L.part, nq, pre)) return false;
  }
  stamp(a, cx, st, TR_QKV_GEMV);
  for (int i = tid_opaque(); i < nq * (r1 - r0); i += BLOCK) {
    const int p = i / (r1 - r0), r = r0 + i % (r1 - r0);
    const float v = L.out[i];
    if (r < SH::QL) ll_put_f32(vbuf(a, a.off.vcqr, SH::QL, p) + r, v, st.k1);
    else ll_put_f32(vbuf(a, a.off.vckv, SH::LAT, p) + (r - SH::QL), v, st.k1);
  }
  stamp(a, cx, st, TR_QKV_DONE);
  return true;
}

// ------------------------------------------------------------------ BQ
template <class SH>
__device__ __forceinline__ bool bstage_q(Ctx& cx, const KArgs& a, const Step& st, VLds& L, int nq) {
  const DLayer Ly = *gp(st.Ly);
  const int w = cx.w, nwg = cx.nwg;
  constexpr int QL = SH::QL, RQ = SH::NH * SH::QH, AST = vb_astr(QL);
  const int r0 = 2 * split_at(RQ / 2, nwg, w), r1 = 2 * split_at(RQ / 2, nwg, w + 1);
  float* tmp = reinterpret_cast<float*>(L.A + VB * AST);   // [VB][QL] fp32
  RegPairs<QL> gq;
  gq.load(Ly.q_norm);
  __syncthreads();
  mseg_set(L.segs, 0, Ly.w_uq.w + (size_t)r0 * QL, Ly.w_uq.s, r1 - r0, r0, 0, 0, nq);
  __syncthreads();
  auto pre = [&]() -> bool {
    if (!ll_fetch_rows<QL>(cx, reinterpret_cast<uint32_t*>(tmp), QL, vbuf(a, a.off.vcqr, QL, 0), QL, nq, st.k1, W_CQ))
      return false;
    rms_rows<QL>(L.A, AST, [&](int p, int j) { return reinterpret_cast<const float2*>(tmp + p * QL)[j]; }, gq, a.c.eps,
                 L.redv, nq);
    stamp(a, cx, st, TR_CQ_READY);
    return true;
  };
  if (!mfma_list<QL, 4>(L.segs, r1 > r0 ? 1 : 0, L.A, L.out, r1 - r0, L.part, nq, pre)) return false;
  stamp(a, cx, st, TR_Q_GEMV);
  const int npair = (r1 - r0) / 2;
  for (int i = tid_opaque(); i < nq * npair; i += BLOCK) {
    const int p = i / npair, r = r0 + 2 * (i % npair), h = r / SH::QH, k = r % SH::QH;
    const float v0 = L.out[p * (r1 - r0) + r - r0], v1 = L.out[p * (r1 - r0) + r + 1 - r0];
    if (k < SH::ND) {
      uint64_t* qn = vbuf(a, a.off.vqn, SH::NH * SH::ND, p) + h * SH::ND + k;
      ll_put_f32(qn, v0, st.k1);
      ll_put_f32(qn + 1, v1, st.k1);
    } else {
      const int d = k - SH::ND;
      const PLD_GLOBAL float* rope = gp(wsp<float>(a, a.off.rope)) + (size_t)L.rpos[p] * SH::RD;
      const float cs = rope[d], sn = rope[d + 1];
      ll_put(vbuf(a, a.off.vqr, SH::NH * SH::RD / 2, p) + (h * SH::RD + d) / 2,
             f32_to_bf16(v0 * cs - v1 * sn) | (f32_to_bf16(v0 * sn + v1 * cs) << 16), st.k1);
    }
  }
  stamp(a, cx, st, TR_ATT_Q);
  return true;
}

// ------------------------------------------------------------------ BA: q_lat = W_UK^T q_nope (per position)
// Workgroup (head h, cpw columns); thread (row group rr, 16-column chunk ck) holds its rows'
// weights in registers for every position. Per position: the thread's partial column sums,
// reduced over the 8 row groups of a wave with lane shuffles, then over the 8 waves in LDS
// (all positions at once).
template <class SH>
__device__ __forceinline__ bool bstage_absorb(Ctx& cx, const KArgs& a, const Step& st, VLds& L, int nq) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  constexpr int EPC = 16, KL = SH::KL, ND = SH::ND;
  constexpr int SBK = (KL + 127) / 128;
  const int cpw = c.cpw;
  const int h = (cx.w * cpw) / KL, c0 = (cx.w * cpw) % KL;
  const int cpr = cpw / EPC, rpp = BLOCK / cpr;   // host: cpw == 128 (8 chunks per row, 64 row groups)
  constexpr int MAXP = 4;
  const int tid = tid_opaque();
  const int lane = tid & 63, wave = tid >> 6;
  const int ck = tid % cpr, rr = tid / cpr;
  uint4 wv[MAXP];
  float sc[MAXP];
#pragma unroll
  for (int p = 0; p < MAXP; p++) {
    wv[p] = make_uint4(0u, 0u, 0u, 0u);
    sc[p] = 0.f;
    if (p * rpp < ND) {
      const int d = min(rr + p * rpp, ND - 1);
      const size_t row = (size_t)h * ND + d;
      wv[p] = ld_stream16(Ly.w_uk.w + row * KL + c0 + ck * EPC);
      sc[p] = gp(Ly.w_uk.s)[(row >> 7) * SBK + ((c0 + ck * EPC) >> 7)];
    }
  }
  float* qv = reinterpret_cast<float*>(L.A);   // [VB][ND] q_nope of head h per position
  float* red = qv + VB * ND;                   // [VB][NWAVES][cpw] wave partial column sums
  if (!ll_fetch_rows<ND>(cx, reinterpret_cast<uint32_t*>(qv), ND, vbuf(a, a.off.vqn, SH::NH * ND, 0) + (size_t)h * ND,
                         SH::NH * ND, nq, st.k1, W_QN))
    return false;
  for (int q = 0; q < nq; q++) {
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; e++) acc[e] = 0.f;
#pragma unroll
    for (int p = 0; p < MAXP; p++) {
      const int d = rr + p * rpp;
      if (p * rpp < ND) {
        const float qq = d < ND ? qv[q * ND + d] * sc[p] : 0.f;
        const uint32_t wd[4] = {wv[p].x, wv[p].y, wv[p].z, wv[p].w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[i], false);
          const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[i], true);
          acc[4 * i + 0] = fmaf(lo.x, qq, acc[4 * i + 0]);
          acc[4 * i + 1] = fmaf(lo.y, qq, acc[4 * i + 1]);
          acc[4 * i + 2] = fmaf(hi.x, qq, acc[4 * i + 2]);
          acc[4 * i + 3] = fmaf(hi.y, qq, acc[4 * i + 3]);
        }
      }
    }
    // the 8 row groups of a wave are lane bits 3..5
#pragma unroll
    for (int e = 0; e < EPC; e++) {
      float v = acc[e];
      v += __shfl_xor(v, 8, 64);
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      acc[e] = v;
    }
    if (lane < 8) {
#pragma unroll
      for (int e = 0; e < EPC; e++) red[(q * NWAVES + wave) * cpw + ck * EPC + e] = acc[e];
    }
  }
  __syncthreads();
  // q_lat as bf16 pairs: the attention's matrix cores take it in bf16 (same rounding)
  for (int i = tid; i < nq * (cpw / 2); i += BLOCK) {
    const int q = i / (cpw / 2), j = 2 * (i % (cpw / 2));
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int wv2 = 0; wv2 < NWAVES; wv2++) {
      s0 += red[(q * NWAVES + wv2) * cpw + j];
      s1 += red[(q * NWAVES + wv2) * cpw + j + 1];
    }
    ll_put(vbuf(a, a.off.vqlat, SH::NH * KL / 2, q) + ((size_t)h * KL + c0 + j) / 2,
           f32_to_bf16(s0) | (f32_to_bf16(s1) << 16), st.k1);
  }
  __syncthreads();
  stamp(a, cx, st, TR_ATT_SCORES);
  return true;
}

// The new latent rows of the step's rows plo .. phi - 1 (computed by the last chunk's
// workgroups): their c_kv' | k_r' fetched together into tmp [VB][LAT] fp32 (LDS), RMSNorm of
// c_kv (fp64 statistics, one reduction for all rows) and RoPE of k_r at each row's position,
// bf16 into newr [VB][LAT]; with append, each row is also written to its cache row crow(p).
template <class SH, typename CRow>
__device__ __forceinline__ bool new_rows(Ctx& cx, const KArgs& a, const DLayer& Ly, VLds& V, int plo, int phi,
                                         uint32_t k1, bool append, float* tmp, uint16_t* newr, CRow&& crow) {
  constexpr int LAT = SH::LAT, KL = SH::KL, RD = SH::RD;
  constexpr int NE = (VB * (LAT / 2) + BLOCK - 1) / BLOCK;   // output pairs per thread
  const int tid = tid_opaque();
  // this thread's RMSNorm weights (c_kv) or RoPE factors (k_r), loaded before the fetch so
  // that they do not wait behind it
  const int nr = phi - plo;
  float f0[NE], f1[NE];
#pragma unroll
  for (int j = 0; j < NE; j++) {
    const int e = min(tid + j * BLOCK, nr * (LAT / 2) - 1), p = plo + e / (LAT / 2), k = 2 * (e % (LAT / 2));
    const PLD_GLOBAL float* src = k < KL ? gp(Ly.kv_norm) + k
                                         : gp(wsp<float>(a, a.off.rope)) + (size_t)V.rpos[p] * RD + (k - KL);
    f0[j] = src[0];
    f1[j] = src[1];
  }
  if (!ll_fetch_rows<LAT>(cx, reinterpret_cast<uint32_t*>(tmp + plo * LAT), LAT, vbuf(a, a.off.vckv, LAT, plo), LAT, nr, k1,
                         W_KV))
    return false;
  double ss[VB];
#pragma unroll
  for (int p = 0; p < VB; p++) {
    ss[p] = 0.0;
    if (p >= plo && p < phi)
      for (int i = tid; i < KL; i += BLOCK) ss[p] += (double)tmp[p * LAT + i] * (double)tmp[p * LAT + i];
  }
  block_sum_rows(ss, V.redv);
#pragma unroll
  for (int p = 0; p < VB; p++) ss[p] = 1.0 / sqrt(ss[p] / (double)KL + a.c.eps);   // each row's norm scale
#pragma unroll
  for (int j = 0; j < NE; j++) {
    const int e = tid + j * BLOCK;
    if (e >= nr * (LAT / 2)) break;
    const int p = plo + e / (LAT / 2), i = e % (LAT / 2), k = 2 * i;
    double r = 0.0;
#pragma unroll
    for (int q = 0; q < VB; q++) r = q == p ? ss[q] : r;   // (ss[] holds the scales, below)
    const float* x = tmp + p * LAT;
    float v0, v1;
    if (k < KL) {
      v0 = (float)(((double)x[k] * r) * (double)f0[j]);
      v1 = (float)(((double)x[k + 1] * r) * (double)f1[j]);
    } else {
      const float x0 = x[k], x1 = x[k + 1], cs = f0[j], sg = f1[j];
      v0 = x0 * cs - x1 * sg;
      v1 = x0 * sg + x1 * cs;
    }
    const uint32_t pair = f32_to_bf16(v0) | (f32_to_bf16(v1) << 16);
    reinterpret_cast<uint32_t*>(newr + p * LAT)[i] = pair;
    if (append) st_u32(reinterpret_cast<uint32_t*>(Ly.lat + crow(p) * LAT) + i, pair);
  }
  __syncthreads();
  vm_wait();   // the appended rows are written before this workgroup's next publication
  return true;
}

// ------------------------------------------------------------------ BT: attention of a batch decode
// Every row is a sequence of its own: its cache rows start at p * max_seq and its history is
// [0, rpos[p]). The workgroups of each of the NG = NH / HPW head groups (HPW = 16 heads,
// nwg / NG workgroups each) are dealt to the sequences, CB = (nwg / NG) / nq consecutive
// workgroups per sequence; workgroup (head group hg, sequence b, chunk c) runs one pipeline
// over the 32-row sub-blocks of chunk c of b's history (staged in LDS, double buffer, DEPTH
// register sets of loads in flight): S = Q C^T and O += P C on the matrix cores, online
// softmax per head; the last chunk adds b's new row on the vector ALU. The head groups of
// one (sequence, chunk) are workgroups hg * (nwg / NG) + i for one i, so they lie on one XCD
// and share the rows through its L2; rows written inside this launch are read coherently.
// Partials per (sequence, head, chunk).
template <class SH>
__device__ __forceinline__ int batch_chunks(int nwg, int nq) {
  return (nwg / (SH::NH / SH::HPW)) / nq;
}

template <class SH>
__device__ __forceinline__ bool bstage_attn(Ctx& cx, const KArgs& a, const Step& st, VLds& V, int nq) {
  const DLayer Ly = *gp(st.Ly);
  const uint32_t k1 = st.k1;
  constexpr int LAT = SH::LAT, KL = SH::KL, HPW = SH::HPW, TB = SH::TB, CSTR = SH::CSTR;
  constexpr int KSTEPS = LAT / 16, KQ = KSTEPS / 4;
  constexpr int CPRW = LAT / 8;
  constexpr int NLD = (TB * CPRW + BLOCK - 1) / BLOCK;
  static_assert(HPW == 2 * NWAVES && KL == 512 && TB == 32, "the batched attention tiling (16 heads per workgroup)");
  constexpr int HS = 2;
  const int tid = tid_opaque();
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hown = wave * HS + ((lane & 63) >> 5);
  const int ngw = cx.nwg / (SH::NH / HPW);   // workgroups per head group
  const int CB = batch_chunks<SH>(cx.nwg, nq);
  const int hg = cx.w / ngw, i = cx.w % ngw;
  const int b = i / CB, ch = i % CB;
  if (b >= nq) {   // (nwg / NG not a multiple of nq: the spare workgroups have no chunk)
    stamp(a, cx, st, TR_ATT_PARTIAL);
    return true;
  }
  const int hbase = hg * HPW;
  const int hist = V.rpos[b];
  const int t0 = split_at(hist, CB, ch), n = split_at(hist, CB, ch + 1) - t0;
  const int nsb = (n + TB - 1) / TB;
  const int fresh = hist - cx.token;   // b's rows >= fresh were appended inside this launch (one per step)
  const uint16_t* lat = Ly.lat + (size_t)b * a.c.max_seq * LAT;
  const bool last = ch == CB - 1;
  // LDS
  uint16_t* Qs = V.A;                                        // [16][CSTR]
  uint16_t* Cs = Qs + 16 * CSTR;                             // [2][TB][CSTR]
  uint16_t* Ps = Cs + 2 * TB * CSTR;                         // [16][TB]
  float* Ssc = reinterpret_cast<float*>(Ps + 16 * TB);       // [4][2][256]
  float* alph = Ssc + 4 * 2 * 256;                           // [16]
  uint16_t* newr = reinterpret_cast<uint16_t*>(alph + 16);   // [VB][LAT] new rows (bf16; row b used)
  float* sn = reinterpret_cast<float*>(newr + VB * LAT);     // [16] new-row scores, then [16][2] (p, alpha)
  float* qtmp = reinterpret_cast<float*>(Cs + TB * CSTR);    // q staging (Cs buffer 1, free until the second sub-block)
  // b's new row (last chunk): RMSNorm(c_kv') and RoPE(k_r'), bf16; appended to b's cache
  // row rpos[b] by head group 0
  if (last) {
    // (Cs buffer 0 is free until the first sub-block is staged)
    if (!new_rows<SH>(cx, a, Ly, V, b, b + 1, k1, hg == 0, reinterpret_cast<float*>(Cs), newr,
                      [&](int p) { return (size_t)p * a.c.max_seq + (size_t)V.rpos[p]; }))
      return false;
  }
  const float scale = 1.0f / sqrtf((float)(SH::ND + SH::RD));
  const int ln = lane & 15, lq = lane >> 4;
  constexpr int DEPTH = 3;
  auto fresh_block = [&](int sb) -> bool {   // does sub-block sb hold a row written in this launch?
    const int lr = min(sb * TB + TB, n) - 1;
    return lr >= 0 && t0 + lr >= fresh;
  };
  uint4 cb[DEPTH][NLD];
  auto issue_k = [&](int set, int sb, auto coh_tag) {
    constexpr bool COH = decltype(coh_tag)::value;
    const bool live = sb < nsb;
#pragma unroll
    for (int k8 = 0; k8 < NLD; k8++) {
      const int idx = min(tid + k8 * BLOCK, TB * CPRW - 1);
      const int r = idx / CPRW, k = idx % CPRW;
      const int t = max(min(sb * TB + r, n - 1), 0);
      const uint16_t* p = live ? lat + (size_t)(t0 + t) * LAT + k * 8 : lat;
      cb[set][k8] = COH ? ld_coh16(p) : ld_g16(p);
    }
  };
  auto issue = [&](int set, int sb) {
    if (sb < nsb && fresh_block(sb)) issue_k(set, sb, std::true_type{});
    else issue_k(set, sb, std::false_type{});
  };
  auto store = [&](int set, int buf) {
    uint16_t* C = Cs + buf * TB * CSTR;
#pragma unroll
    for (int k8 = 0; k8 < NLD; k8++) {
      const int idx = tid + k8 * BLOCK;
      if (idx < TB * CPRW) {
        const int r = idx / CPRW, k = idx % CPRW;
        uint32_t* d = reinterpret_cast<uint32_t*>(C + r * CSTR + k * 8);
        d[0] = cb[set][k8].x; d[1] = cb[set][k8].y; d[2] = cb[set][k8].z; d[3] = cb[set][k8].w;
      }
    }
  };
#pragma unroll
  for (int d = 0; d < DEPTH; d++) issue(d, d);
  // b's queries: q_lat [HPW][KL] and q_rope [HPW][RD] (bf16 pairs) -> rows of Qs
  {
    constexpr int RD = SH::RD;
    uint32_t* qw = reinterpret_cast<uint32_t*>(qtmp);
    if (!ll_fetch<per_for(HPW * KL / 2)>(cx, qw, vbuf(a, a.off.vqlat, SH::NH * KL / 2, b) + (size_t)hbase * KL / 2,
                                         HPW * KL / 2, k1, W_QLAT))
      return false;
    if (!ll_fetch<per_for(HPW * RD / 2)>(cx, qw + HPW * KL / 2, vbuf(a, a.off.vqr, SH::NH * RD / 2, b) + (size_t)hbase * RD / 2,
                                         HPW * RD / 2, k1, W_QLAT))
      return false;
    for (int e = tid; e < 16 * LAT / 2; e += BLOCK) {
      const int hh = e / (LAT / 2), k2 = e % (LAT / 2);
      const uint32_t v = k2 < KL / 2 ? qw[hh * (KL / 2) + k2] : qw[HPW * KL / 2 + hh * (RD / 2) + (k2 - KL / 2)];
      reinterpret_cast<uint32_t*>(Qs + hh * CSTR)[k2] = v;
    }
    __syncthreads();
  }
  stamp(a, cx, st, TR_ATT_READY);
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 O[4];
#pragma unroll
  for (int t = 0; t < 4; t++) O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto block = [&](const uint16_t* C, int tb0) {
    // S partials: wave pair (wave >> 1) covers k-steps [kq*KQ, +KQ), tile nt = wave & 1
    {
      const int nt = wave & 1, kq = wave >> 1;
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
    // online softmax: head hown, token tb0 + (lane & 31)
    {
      const int tl = lane & 31;
      float s = -INFINITY;
      if (tb0 + tl < n) {
        const int nt = tl >> 4, col = tl & 15;
        s = 0.f;
#pragma unroll
        for (int kq = 0; kq < 4; kq++) s += Ssc[(kq * 2 + nt) * 256 + hown * 16 + col];
        s *= scale;
      }
      const float mb = half_max_dpp(s);
      const float mnew = fmaxf(m_run, mb);
      const float al = m_run == -INFINITY ? 0.f : __expf(m_run - mnew);
      const float pv = s == -INFINITY ? 0.f : __expf(s - mnew);
      l_run = l_run * al + half_sum_dpp(pv);
      m_run = mnew;
      Ps[hown * TB + tl] = (uint16_t)bf16_bits(pv);
      if (tl == 0) alph[hown] = al;
    }
    __syncthreads();
    // O = alpha O + P C: wave owns columns [wave*64, +64)
    float fa[4];
#pragma unroll
    for (int q = 0; q < 4; q++) fa[q] = alph[4 * lq + q];
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
  };
  for (int sb0 = 0; sb0 < nsb; sb0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; d++) {
      const int sb = sb0 + d;
      if (sb >= nsb) break;
      const int buf = sb & 1;
      store(d, buf);
      __syncthreads();
      issue(d, sb + DEPTH);
      block(Cs + buf * TB * CSTR, sb * TB);
    }
  }
  __syncthreads();
  // b's new row (last chunk): thread (half-wave hr = head, lane jj) over LAT / 32 dims
  if (last) {
    constexpr int DPJ = LAT / 32;
    const int hr = tid >> 5, jj = tid & 31;
    const uint16_t* nr = newr + b * LAT;
    float sv = 0.f;
#pragma unroll
    for (int d = 0; d < DPJ; d++) sv = fmaf(bf16_to_f32(Qs[hr * CSTR + jj * DPJ + d]), bf16_to_f32(nr[jj * DPJ + d]), sv);
    sv = dpp_sum<32>(sv);
    if (jj == 31) sn[hr] = sv * scale;
    __syncthreads();
    const float s = sn[hown];
    const float mnew = fmaxf(m_run, s);
    const float al = m_run == -INFINITY ? 0.f : __expf(m_run - mnew);
    const float pr = __expf(s - mnew);
    l_run = l_run * al + pr;
    m_run = mnew;
    if ((lane & 31) == 0) {
      sn[16 + 2 * hown] = pr;
      sn[16 + 2 * hown + 1] = al;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; t++) {
      const int col = (wave * 4 + t) * 16 + ln;
      const float c = bf16_to_f32(nr[col]);
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int hh = 4 * lq + q;
        O[t][q] = fmaf(sn[16 + 2 * hh], c, O[t][q] * sn[16 + 2 * hh + 1]);
      }
    }
  }
  stamp(a, cx, st, TR_ATT_SOFTMAX);
  // publish: m, l (fp32) and the accumulators as fp16 pairs, at (b, head, chunk)
  constexpr int PSTR = vp_stride<KL>();
  uint64_t* pp = wsp<uint64_t>(a, a.off.vpart) + (size_t)b * SH::NH * CB * PSTR;
  if ((lane & 31) == 0) {
    uint64_t* q = pp + ((size_t)(hbase + hown) * CB + ch) * PSTR;
    ll_put_f32(q, m_run, k1);
    ll_put_f32(q + 1, l_run, k1);
  }
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const int col = (wave * 4 + t) * 16 + ln;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const float nb = dpp_mov<0xB1, 0xf, false>(O[t][q]);
      const int hh = 4 * lq + q;
      if ((ln & 1) == 0) {
        const uint32_t pr = (uint32_t)__half_as_ushort(__float2half_rn(O[t][q])) |
                            ((uint32_t)__half_as_ushort(__float2half_rn(nb)) << 16);
        ll_put(pp + ((size_t)(hbase + hh) * CB + ch) * PSTR + VP_ACC + col / 2, pr, k1);
      }
    }
  }
  __syncthreads();
  stamp(a, cx, st, TR_ATT_PARTIAL);
  return true;
}

// ------------------------------------------------------------------ BV: attention of a verify, all positions in one pass
// For the verify (the rows are consecutive positions of one sequence sharing its history):
// workgroup (group of 8 heads, chunk of the history; NG = 8 groups x NCV = nwg / 8 chunks,
// the groups of one chunk on one XCD). The A operand rows are (position, head) pairs, two
// positions per 16-row tile (rows 8 (p & 1) + h of tile p >> 1), so every staged 32-row
// sub-block serves all positions at once: S = Q C^T with wave w on tile (w >> 1, column
// half w & 1) over all 18 k-steps of 32, online softmax per row (8 lanes per row, four columns
// each), O += P C with wave w owning output columns [64 w, 64 w + 64) of all tiles. The last
// chunk adds the new rows of the step as one more sub-block with the causal mask (position p
// sees new rows 0..p). Partials per (position, head, chunk) with NCV chunks.
constexpr int VHG = 8;   // heads per workgroup in the verify attention
template <class SH>
__device__ __forceinline__ bool bstage_attn_v(Ctx& cx, const KArgs& a, const Step& st, VLds& V, int nq) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  const uint32_t k1 = st.k1;
  constexpr int LAT = SH::LAT, KL = SH::KL, RD = SH::RD, TB = SH::TB;
  constexpr int CSTR = LAT + 8;   // LDS row stride (bf16): rows 16-byte aligned for the 16-byte operand reads
  constexpr int KSTEPS = LAT / 32;
  constexpr int CPRW = LAT / 8;
  constexpr int NLD = (TB * CPRW + BLOCK - 1) / BLOCK;
  constexpr int MT = VB / 2;            // 16-row tiles of (position, head) rows
  constexpr int QW = KL / 2 + RD / 2;   // words of one (position, head) query row
  static_assert(KL == 512 && TB == 32 && SH::NH % VHG == 0 && NWAVES == 2 * MT, "the verify attention tiling");
  static_assert(LAT % 32 == 0, "whole 32-wide k-steps");
  // LDS: Qs, Cs, Ps, Ssc, alph, newr, ntmp, sn (below) inside the operand region
  static_assert((MT * 16 + TB) * CSTR * 2 + MT * 16 * TB * 2 + (MT * 2 * 256 + MT * 16) * 4 + VB * LAT * 2 + LAT * 4 +
                        MT * 16 * (VB + 2) * 4 <= VACT_BYTES,
                "verify attention LDS");
  const int tid = tid_opaque();
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15, lq = lane >> 4;
  const int nch = cx.nwg / (SH::NH / VHG);   // chunks per head group
  const int hg = cx.w / nch, ch = cx.w % nch;
  const int hbase = hg * VHG;
  const int pos = V.rpos[0];                 // history rows [0, pos), shared by all positions
  // the split counts the last chunk's extra work as 3 TB more rows (its new-row sub-block,
  // and the new rows' norm and RoPE, which take about two sub-blocks' time), so that chunk
  // holds about three history sub-blocks fewer and finishes with the others
  constexpr int XTRA = 3 * TB;
  const int t0 = split_at(pos + XTRA, nch, ch), n = max(0, min(split_at(pos + XTRA, nch, ch + 1), pos) - t0);
  const uint16_t* lat = Ly.lat;
  // LDS
  uint16_t* Qs = V.A;                                        // [MT * 16][CSTR] (position, head) rows
  uint16_t* Cs = Qs + MT * 16 * CSTR;                        // [TB][CSTR] the staged sub-block
  uint16_t* Ps = Cs + TB * CSTR;                             // [MT * 16][TB] bf16
  float* Ssc = reinterpret_cast<float*>(Ps + MT * 16 * TB);  // [MT][2][256] score tiles
  float* alph = Ssc + MT * 2 * 256;                          // [MT * 16]
  uint16_t* newr = reinterpret_cast<uint16_t*>(alph + MT * 16);   // [VB][LAT] new rows (bf16)
  float* ntmp = reinterpret_cast<float*>(newr + VB * LAT);   // [LAT]
  float* sn = ntmp + LAT;                                    // [MT * 16][VB + 2] new-row scores, p, alpha
  const bool last = ch == nch - 1;
  // sub-block staging: DEPTH register sets, loads issued DEPTH blocks ahead (static rows: L2)
  const int nsb = (n + TB - 1) / TB;
  constexpr int DEPTH = 2;
  uint4 cb[DEPTH][NLD];
  auto issue = [&](int set, int sb) {
    const bool live = sb < nsb;
#pragma unroll
    for (int i = 0; i < NLD; i++) {
      const int idx = min(tid + i * BLOCK, TB * CPRW - 1);
      const int r = idx / CPRW, k = idx % CPRW;
      const int t = max(min(sb * TB + r, n - 1), 0);
      const uint16_t* p = live ? lat + (size_t)(t0 + t) * LAT + k * 8 : lat;
      cb[set][i] = ld_g16(p);
    }
  };
#pragma unroll
  for (int d = 0; d < DEPTH; d++) issue(d, d);
  // queries of all positions: q_lat [8 heads][KL] then q_rope [8 heads][RD] (bf16 pairs) -> Qs
  // rows; one LL fetch (word (p, h, k2) of the query row lands at Qs row (p, h), word k2)
  {
    const int qlat_off = (int)((a.off.vqlat - a.off.vqr) / 8);   // vqlat lies after vqr
    struct IdxQ {
      int qlat_off, hbase;
      __device__ __forceinline__ int operator()(int i) const {
        const int p = i / (VHG * QW), k = i % (VHG * QW);
        if (k < VHG * (KL / 2)) return qlat_off + p * (SH::NH * KL / 2) + hbase * (KL / 2) + k;
        const int j = k - VHG * (KL / 2);
        return p * (SH::NH * RD / 2) + hbase * (RD / 2) + j;
      }
    };
    struct StQ {
      __device__ __forceinline__ void operator()(uint32_t* dst, int i, uint32_t v) const {
        const int p = i / (VHG * QW), k = i % (VHG * QW);
        int h, k2;
        if (k < VHG * (KL / 2)) {
          h = k / (KL / 2);
          k2 = k % (KL / 2);
        } else {
          const int j = k - VHG * (KL / 2);
          h = j / (RD / 2);
          k2 = KL / 2 + j % (RD / 2);
        }
        dst[(((p >> 1) * 16 + (p & 1) * VHG + h) * CSTR) / 2 + k2] = v;
      }
    };
    for (int i = tid; i < (MT * 16 - nq * VHG) * (CSTR / 2); i += BLOCK)   // rows of absent positions: zero
      reinterpret_cast<uint32_t*>(Qs)[nq * VHG * (CSTR / 2) + i] = 0u;
    if (!ll_fetch<per_for(VB * VHG * QW)>(cx, reinterpret_cast<uint32_t*>(Qs), wsp<uint64_t>(a, a.off.vqr),
                                          nq * VHG * QW, k1, W_QLAT, IdxQ{qlat_off, hbase}, StQ{}))
      return false;
  }
  // the new rows of this step (last chunk): RMSNorm(c_kv') and RoPE(k_r'), bf16; appended by group 0
  if (last) {
    // (after the queries, which every chunk waits for: the new rows' input was published
    // long before; Cs is free until the first sub-block is staged, and the first sub-blocks'
    // loads, issued above, are in flight meanwhile)
    if (!new_rows<SH>(cx, a, Ly, V, 0, nq, k1, hg == 0, reinterpret_cast<float*>(Cs), newr,
                      [&](int p) { return (size_t)V.rpos[p]; }))
      return false;
  }
  for (int i = tid; i < MT * 16 * TB; i += BLOCK) Ps[i] = 0;
  __syncthreads();
  stamp(a, cx, st, TR_ATT_READY);
  const float scale = 1.0f / sqrtf((float)(SH::ND + SH::RD));
  // softmax: thread t owns row R = t / 8 of the MT * 16 (position, head) rows and four of
  // the sub-block's 32 columns; its row's running max and sum (the same in its 8 lanes)
  const int srow = tid >> 3, scg = tid & 7, smi = srow >> 4, sr16 = srow & 15;
  const int sprow = 2 * smi + (sr16 >= VHG ? 1 : 0);   // the row's position
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 O[MT][4];
#pragma unroll
  for (int mi = 0; mi < MT; mi++) {
#pragma unroll
    for (int t = 0; t < 4; t++) O[mi][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto row_live = [&](int mi, int r16) { return 2 * mi + (r16 >= VHG ? 1 : 0) < nq; };
  auto block = [&](int tb0, bool causal) {
    // S tile (mi, nt) of wave w: two accumulator chains over the 18 k-steps of 32 (lane
    // (ln, lq) supplies k = 8 lq .. 8 lq + 7 of its row for both operands)
    {
      const int mi = wave >> 1, nt = wave & 1;
      f32x4 s4 = {0.f, 0.f, 0.f, 0.f}, s5 = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* Q = Qs + mi * 16 * CSTR;
      if (2 * mi < nq) {   // (a tile with no live row is masked by the softmax: not computed)
#pragma unroll
        for (int kk = 0; kk < KSTEPS; kk++) {
          const int k0 = kk * 32 + 8 * lq;
          const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(Q + ln * CSTR + k0);
          const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(Cs + (nt * 16 + ln) * CSTR + k0);
          if (kk & 1) s5 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, s5, 0, 0, 0);
          else s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, s4, 0, 0, 0);
        }
      }
      s4 += s5;
      float* dst = Ssc + (mi * 2 + nt) * 256;
#pragma unroll
      for (int q = 0; q < 4; q++) dst[(4 * lq + q) * 16 + ln] = s4[q];
    }
    __syncthreads();
    // online softmax of row srow over tokens tb0 + 4 scg .. + 3 (causal: new rows, row
    // position p sees new rows 0..p); max and sum over the row's 8 lanes with DPP moves
    {
      const float4 sv = *reinterpret_cast<const float4*>(Ssc + (smi * 2 + (scg >> 2)) * 256 + sr16 * 16 + 4 * (scg & 3));
      float sc[4] = {sv.x, sv.y, sv.z, sv.w};
      float mb = -INFINITY;
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const int tl = 4 * scg + c;
        const bool ok = (causal ? (tl < nq && tl <= sprow) : (tb0 + tl < n)) && sprow < nq;
        sc[c] = ok ? sc[c] * scale : -INFINITY;
        mb = fmaxf(mb, sc[c]);
      }
      mb = fmaxf(mb, dpp_mov<0xB1, 0xf, false>(mb));    // quad_perm [1,0,3,2]
      mb = fmaxf(mb, dpp_mov<0x4E, 0xf, false>(mb));    // quad_perm [2,3,0,1]
      mb = fmaxf(mb, dpp_mov<0x141, 0xf, false>(mb));   // row_half_mirror: max of 8
      const float mnew = fmaxf(m_run, mb);
      const float al = m_run == -INFINITY ? 0.f : __expf(m_run - mnew);
      float ps = 0.f;
      uint32_t pb[4];
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const float pv = sc[c] == -INFINITY ? 0.f : __expf(sc[c] - mnew);
        ps += pv;
        pb[c] = (uint32_t)(uint16_t)bf16_bits(pv);
      }
      l_run = l_run * al + dpp_sum<8>(ps);
      m_run = mnew;
      *reinterpret_cast<uint2*>(Ps + srow * TB + 4 * scg) = make_uint2(pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16));
      if (scg == 0) alph[srow] = al;
    }
    __syncthreads();
    // O = alpha O + P C: wave owns columns [wave*64, +64) of every tile, one 16x16x32 product
    // per (tile, column tile) over the sub-block's 32 rows (lane (ln, lq) supplies rows
    // 8 lq .. 8 lq + 7 of both operands); tiles with no live row (positions >= nq) are skipped
#pragma unroll
    for (int mi = 0; mi < MT; mi++) {
      if (2 * mi < nq) {
        float fa[4];
#pragma unroll
        for (int q = 0; q < 4; q++) fa[q] = alph[mi * 16 + 4 * lq + q];
#pragma unroll
        for (int t = 0; t < 4; t++)
#pragma unroll
          for (int q = 0; q < 4; q++) O[mi][t][q] *= fa[q];
      }
    }
    static_assert(TB == 32, "one 32-deep product per sub-block");
    bf16x8_t av[MT];
#pragma unroll
    for (int mi = 0; mi < MT; mi++) av[mi] = *reinterpret_cast<const bf16x8_t*>(Ps + (mi * 16 + ln) * TB + 8 * lq);
#pragma unroll
    for (int t = 0; t < 4; t++) {
      const int col = (wave * 4 + t) * 16 + ln;
      uint32_t bw[4];
#pragma unroll
      for (int q = 0; q < 4; q++)
        bw[q] = (uint32_t)Cs[(8 * lq + 2 * q) * CSTR + col] | ((uint32_t)Cs[(8 * lq + 2 * q + 1) * CSTR + col] << 16);
      const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, make_uint4(bw[0], bw[1], bw[2], bw[3]));
#pragma unroll
      for (int mi = 0; mi < MT; mi++)
        if (2 * mi < nq) O[mi][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mi], bv, O[mi][t], 0, 0, 0);
    }
  };
  // the history sub-blocks, then (last chunk) the new rows of the step as one more sub-block
  // with the causal mask: row (p, h) sees new rows 0..p
  const int nall = nsb + (last ? 1 : 0);
  for (int sb0 = 0; sb0 < nall; sb0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; d++) {
      const int sb = sb0 + d;
      if (sb >= nall) break;
      __syncthreads();   // (the previous block's reads of Cs are done)
      if (sb < nsb) {
#pragma unroll
        for (int i = 0; i < NLD; i++) {
          const int idx = tid + i * BLOCK;
          if (idx < TB * CPRW) {
            const int r = idx / CPRW, k = idx % CPRW;
            *reinterpret_cast<uint4*>(Cs + r * CSTR + k * 8) = cb[d][i];   // (16-byte aligned rows)
          }
        }
      } else {
        for (int i = tid; i < TB * (CSTR / 2); i += BLOCK) {
          const int r = i / (CSTR / 2), k2 = i % (CSTR / 2);
          reinterpret_cast<uint32_t*>(Cs)[i] =
              (r < nq && k2 < LAT / 2) ? reinterpret_cast<const uint32_t*>(newr + r * LAT)[k2] : 0u;
        }
      }
      __syncthreads();
      issue(d, sb + DEPTH);
      block(sb * TB, sb >= nsb);
    }
  }
  __syncthreads();
  stamp(a, cx, st, 17);
  stamp(a, cx, st, TR_ATT_SOFTMAX);
  // partials of (position p, head hbase + h, chunk), whole 128-byte lines per store
  // instruction: the (m, l) line from the row's 8 lanes (m, l, then zeros), and the acc words
  // of a tile pair (2u, 2u + 1) as 16 consecutive words per row: the even lanes of a row
  // write tile 2u's pairs (columns ln, ln + 1), the odd lanes tile 2u + 1's (ln - 1, ln)
  constexpr int PSTR = vp_stride<KL>();
  const size_t pwords = (size_t)SH::NH * c.cpg * PSTR;   // per-position stride of the partial buffer
  uint64_t* pll = wsp<uint64_t>(a, a.off.vpart);
  if (sprow < nq) {
    uint64_t* q = pll + (size_t)sprow * pwords + ((size_t)(hbase + (sr16 & (VHG - 1))) * nch + ch) * PSTR + 2 * scg;
    ll_put_f32(q, scg == 0 ? m_run : 0.f, k1);
    ll_put_f32(q + 1, scg == 0 ? l_run : 0.f, k1);
  }
  const bool ev = (ln & 1) == 0;
#pragma unroll
  for (int mi = 0; mi < MT; mi++) {
#pragma unroll
    for (int u = 0; u < 2; u++) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const float a0 = O[mi][2 * u][q], a1 = O[mi][2 * u + 1][q];
        const float n0 = dpp_mov<0xB1, 0xf, false>(a0), n1 = dpp_mov<0xB1, 0xf, false>(a1);   // lane ln ^ 1
        const float lo = ev ? a0 : n1, hi = ev ? n0 : a1;
        const int r16 = 4 * lq + q, p = 2 * mi + (r16 >= VHG ? 1 : 0), h = r16 & (VHG - 1);
        if (p < nq) {
          const uint32_t pr = (uint32_t)__half_as_ushort(__float2half_rn(lo)) |
                              ((uint32_t)__half_as_ushort(__float2half_rn(hi)) << 16);
          const int word = (wave * 4 + 2 * u) * 8 + (ev ? 0 : 8) + (ln >> 1);
          ll_put(pll + (size_t)p * pwords + ((size_t)(hbase + h) * nch + ch) * PSTR + VP_ACC + word, pr, k1);
        }
      }
    }
  }
  stamp(a, cx, st, TR_ATT_PARTIAL);
  return true;
}

// ------------------------------------------------------------------ BM: merge, per position
// Workgroup (head h, cpw columns) as in the single-position stage; the partials of MG
// positions (all eight when they fit in LDS, else four) are fetched together (one LL
// fetch), then wave p (< MG) forms position p's
// chunk weights and thread (p, column) sums the chunks.
template <class SH>
__device__ __forceinline__ bool bstage_merge(Ctx& cx, const KArgs& a, const Step& st, VLds& V, int nq) {
  const KCfg& c = a.c;
  constexpr int KL = SH::KL;
  // chunks per head: the verify attention's (8 heads per workgroup) or a batch sequence's
  const int nch = a.bmode == 0 ? cx.nwg / (SH::NH / VHG) : batch_chunks<SH>(cx.nwg, nq), cpw = c.cpw;
  const int MG = (size_t)NWAVES * (nch * (cpw + 3) + 1) * 4 <= (size_t)VACT_BYTES ? NWAVES : NWAVES / 2;
  const int h = (cx.w * cpw) / KL, c0 = (cx.w * cpw) % KL;
  const int tid = tid_opaque();
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int PSTR = vp_stride<KL>();
  const int cpw2 = cpw / 2, nacc = nch * cpw, naw = nch * cpw2;
  const int per = naw + 2 * nch;                 // words of one position
  const int pwords = SH::NH * (a.bmode == 0 ? c.cpg : nch) * PSTR;   // LL words of one position's partials (stride)
  const int fstr = nacc + 2 * nch;               // floats of one position in LDS
  // word i of the group: position i / per, then as in the single-position stage
  struct IdxM {
    int per, naw, cpw2, nch, h, c0, pwords;
    __device__ __forceinline__ int operator()(int i) const {
      const int q = i / per, k = i % per;
      if (k < naw) return q * pwords + (h * nch + k / cpw2) * PSTR + VP_ACC + c0 / 2 + k % cpw2;
      const int j = k - naw;
      return q * pwords + (h * nch + (j >> 1)) * PSTR + (j & 1);
    }
  };
  struct StM {
    int per, naw, fstr;
    __device__ __forceinline__ void operator()(uint32_t* dst, int i, uint32_t v) const {
      const int q = i / per, k = i % per;
      uint32_t* d = dst + q * fstr;
      if (k < naw) {
        reinterpret_cast<float2*>(d)[k] = make_float2(__half2float(__ushort_as_half((unsigned short)(v & 0xffffu))),
                                                      __half2float(__ushort_as_half((unsigned short)(v >> 16))));
      } else {
        d[naw + k] = v;
      }
    }
  };
  float* base = reinterpret_cast<float*>(V.A);     // [MG][nacc floats, then (m, l) per chunk]
  float* fw = base + MG * fstr;                    // [MG][nch]
  float* lsum = fw + MG * nch;                     // [MG]
  stamp(a, cx, st, TR_MERGE_START);
  for (int p0 = 0; p0 < nq; p0 += MG) {
    const int np = min(MG, nq - p0);
    if (!ll_fetch<24>(cx, reinterpret_cast<uint32_t*>(base), wsp<uint64_t>(a, a.off.vpart) + (size_t)p0 * pwords,
                      np * per, st.k1, W_PART, IdxM{per, naw, cpw2, nch, h, c0, pwords}, StM{per, naw, fstr}))
      return false;
    if (p0 == 0) stamp(a, cx, st, TR_MERGE_COPIED);
    if (wave < np) {
      const float* mls = base + wave * fstr + nacc;
      float M = -INFINITY;
      for (int cc = lane; cc < nch; cc += 64)
        if (mls[2 * cc + 1] > 0.f) M = fmaxf(M, mls[2 * cc]);
      M = wave_max_dpp(M);
      float ls = 0.f;
      for (int cc = lane; cc < nch; cc += 64) {
        const float l = mls[2 * cc + 1];
        const float f = l > 0.f ? __expf(mls[2 * cc] - M) : 0.f;
        fw[wave * nch + cc] = f;
        ls += f * l;
      }
      ls = wave_sum_dpp(ls);
      if (lane == 0) lsum[wave] = ls;
    }
    __syncthreads();
    for (int i = tid; i < np * cpw; i += BLOCK) {
      const int q = i / cpw, j = i % cpw;
      const float* accs = base + q * fstr;
      float o = 0.f;
      for (int cc = 0; cc < nch; cc++) o = fmaf(fw[q * nch + cc], accs[cc * cpw + j], o);
      ll_put_f32(vbuf(a, a.off.volat, SH::NH * KL, p0 + q) + (size_t)h * KL + c0 + j, o / lsum[q], st.k1);
    }
    __syncthreads();
  }
  stamp(a, cx, st, TR_ATT_MERGED);
  return true;
}

// ------------------------------------------------------------------ BU: o = W_UV o_lat (matrix cores)
template <class SH>
__device__ __forceinline__ bool bstage_uv(Ctx& cx, const KArgs& a, const Step& st, VLds& L, int nq) {
  const DLayer Ly = *gp(st.Ly);
  constexpr int R = SH::NH * SH::VD, KL = SH::KL, AST = vb_astr(KL);
  const int r0 = split_at(R, cx.nwg, cx.w), r1 = split_at(R, cx.nwg, cx.w + 1);
  const int h = r0 / SH::VD;   // host: every workgroup's rows lie in one head, an even count
  float* tmp = reinterpret_cast<float*>(L.A + VB * AST);
  __syncthreads();
  mseg_set(L.segs, 0, Ly.w_uv.w + (size_t)r0 * KL, Ly.w_uv.s, r1 - r0, r0, 0, 0, nq);
  __syncthreads();
  auto pre = [&]() -> bool {
    if (!ll_fetch_rows<KL>(cx, reinterpret_cast<uint32_t*>(tmp), KL, vbuf(a, a.off.volat, SH::NH * KL, 0) + (size_t)h * KL,
                           SH::NH * KL, nq, st.k1, W_OLAT))
      return false;
    for (int i = tid_opaque(); i < nq * KL; i += BLOCK) L.A[(i / KL) * AST + i % KL] = (uint16_t)f32_to_bf16(tmp[i]);
    __syncthreads();
    return true;
  };
  if (!mfma_list<KL, 2>(L.segs, r1 > r0 ? 1 : 0, L.A, L.out, r1 - r0, L.part, nq, pre)) return false;
  const int npair = (r1 - r0) / 2;
  for (int i = tid_opaque(); i < nq * npair; i += BLOCK) {
    const int p = i / npair, r = r0 + 2 * (i % npair);
    ll_put(vbuf(a, a.off.vo, R / 2, p) + r / 2,
           f32_to_bf16(L.out[p * (r1 - r0) + r - r0]) | (f32_to_bf16(L.out[p * (r1 - r0) + r + 1 - r0]) << 16), st.k1);
  }
  stamp(a, cx, st, TR_ATT_DONE);
  return true;
}

// ------------------------------------------------------------------ BO: h2 = x + W_O o (matrix cores)
template <class SH>
__device__ __forceinline__ bool bstage_wo(Ctx& cx, const KArgs& a, const Step& st, VLds& L, int nq) {
  constexpr int OD = SH::ODIM, AST = vb_astr(OD);
  int r0, r1;
  hrows(SH::H, cx.nwg, cx.w, &r0, &r1);
  const DLayer Ly = *gp(st.Ly);
  const KCfg& c = a.c;
  const int tid = tid_opaque(), nr = r1 - r0;
  __syncthreads();
  mseg_set(L.segs, 0, Ly.wo.w + (size_t)r0 * OD, Ly.wo.s, nr, r0, 0, 0, nq);
  __syncthreads();
  // loaded ahead of the W_O stream: thread (half hh, expert e) takes its half of the row
  // pairs of W_r[e][r0, r1) (bf16 pairs); thread (p, r) the FFN norm weight gamma[r0 + r]
  constexpr int RW = 8;   // pairs per half: rows per workgroup <= 32
  const int np2 = nr / 2, hh = tid >> 8, jb = hh ? np2 / 2 : 0, jn = hh ? np2 - np2 / 2 : np2 / 2;
  uint32_t rw[RW];
  {
    const PLD_GLOBAL uint32_t* rp =
        gp(reinterpret_cast<const uint32_t*>(Ly.router + (size_t)min(tid & 255, c.E - 1) * SH::H + r0)) + jb;
#pragma unroll
    for (int j = 0; j < RW; j++) rw[j] = rp[max(min(j, jn - 1), 0)];
  }
  const float gr = gp(Ly.ffn_norm)[r0 + min(tid & 31, nr - 1)];
  auto pre = [&]() -> bool {
    if (!ll_fetch_rows<OD / 2>(cx, reinterpret_cast<uint32_t*>(L.A), AST / 2, vbuf(a, a.off.vo, OD / 2, 0), OD / 2, nq,
                               st.k1, W_O))
      return false;
    stamp(a, cx, st, TR_O_READY);
    return true;
  };
  if (!mfma_list<OD, 4>(L.segs, nr > 0 ? 1 : 0, L.A, L.out, nr, L.part, nq, pre)) return false;
  // (the A rows are free again: mfma_list ends with a barrier)
  for (int i = tid; i < nq * nr; i += BLOCK) {
    const int p = i / nr, r = i % nr;
    L.h2res[p * 32 + r] = L.xres[p * 32 + r] + L.out[i];
  }
  __syncthreads();
  // This workgroup's share of the FFN norm statistics, sum of h2[p][r]^2 over its rows, one
  // 16-word line [position][lo, hi] written by one store instruction; published first, so
  // that the consumers' norm scale does not wait for the router sums below.
  if (tid < 2 * VB) {
    const int p = tid >> 1;
    double q = 0.0;
    if (p < nq)
      for (int r = 0; r < nr; r++) q += (double)L.h2res[p * 32 + r] * (double)L.h2res[p * 32 + r];
    const uint64_t b = (uint64_t)__double_as_longlong(q);
    ll_put(wsp<uint64_t>(a, a.off.vss) + (size_t)cx.w * VB * 2 + tid, (uint32_t)(b >> (32 * (tid & 1))), st.k1);
  }
  for (int i = tid; i < nq * nr; i += BLOCK) {
    const int p = i / nr, r = i % nr;
    ll_put_f32(vbuf(a, a.off.vh2, SH::H, p) + r0 + r, L.h2res[p * 32 + r], st.k1);
  }
  // the router's partial dot products of expert e over these rows, gamma included:
  // sum_r W_r[e][r0 + r] * gamma[r0 + r] * h2[p][r] (fp64), each half of the rows on its own
  // thread; the router workgroup of e adds the workgroups' sums and applies the norm scale
  double* gh = reinterpret_cast<double*>(L.A);   // [VB][32] gamma_r * h2[p][r] (exact fp64 products)
  double* rpl = gh + VB * 32;                    // [2][256][VB] the two halves' sums
  if (tid < VB * 32) {
    const int p = tid >> 5, r = tid & 31;
    gh[tid] = (p < nq && r < nr) ? (double)gr * (double)L.h2res[p * 32 + r] : 0.0;
  }
  __syncthreads();
  if ((tid & 255) < c.E) {
    double acc[VB];
#pragma unroll
    for (int p = 0; p < VB; p++) acc[p] = 0.0;
#pragma unroll
    for (int j = 0; j < RW; j++) {
      if (j < jn) {
        const int r = 2 * (jb + j);
        const double w0 = (double)bf_lo(rw[j]), w1 = (double)bf_hi(rw[j]);
        double g0[VB], g1[VB];
#pragma unroll
        for (int p = 0; p < VB; p++) {
          g0[p] = gh[p * 32 + r];
          g1[p] = gh[p * 32 + r + 1];
        }
#pragma unroll
        for (int p = 0; p < VB; p++) acc[p] = fma(w1, g1[p], fma(w0, g0[p], acc[p]));
      }
    }
#pragma unroll
    for (int p = 0; p < VB; p++) rpl[(hh * 256 + (tid & 255)) * VB + p] = acc[p];
  }
  __syncthreads();
  // Published as whole 128-byte lines: the 16 words [position][lo, hi] of (expert e, this
  // workgroup) come from 16 consecutive lanes (scattered 8-byte stores from every workgroup
  // would each be a separate partial-line write to memory).
  {
    uint64_t* rpb = wsp<uint64_t>(a, a.off.vrp);
    const int k = tid & 15, p = k >> 1;
    for (int e = tid >> 4; e < c.E; e += BLOCK / 16) {
      const double v = p < nq ? rpl[e * VB + p] + rpl[(256 + e) * VB + p] : 0.0;
      const uint64_t b = (uint64_t)__double_as_longlong(v);
      ll_put(rpb + ((size_t)e * cx.nwg + cx.w) * VB * 2 + k, (uint32_t)(b >> (32 * (k & 1))), st.k1);
    }
  }
  stamp(a, cx, st, TR_WO_DONE);
  // The FFN norm scale of every position, r_p = 1 / sqrt(sum(h2_p^2) / H + eps), from all
  // workgroups' sums (fetched while the router sums above were formed; added in a fixed
  // order: lane sums in producer order, then the wave's tree). It stays in LDS (vnorm) for
  // the FFN stage. Then this workgroup's rows of the FFN operand, bf16(fp32((h2 * r_p) *
  // gamma)), go out as LL words of bf16 pairs: the consumers fetch half the words of fp32 h2
  // and no longer normalise.
  {
    struct IdxS {
      int nq2;
      __device__ __forceinline__ int operator()(int i) const { return (i / nq2) * (VB * 2) + i % nq2; }
    };
    const double* pd = rpl + 2 * 256 * VB;   // [nwg][nq] (fetched fp64 pairs)
    if (!ll_fetch<per_for(256 * VB * 2)>(cx, reinterpret_cast<uint32_t*>(const_cast<double*>(pd)),
                                         wsp<uint64_t>(a, a.off.vss), cx.nwg * nq * 2, st.k1, W_H2, IdxS{nq * 2}))
      return false;
    const int lane = tid & 63, wave = tid >> 6;
    if (wave < nq) {
      double q = 0.0;
      for (int k = lane; k < cx.nwg; k += 64) q += pd[k * nq + wave];
      q = wave_sum_any(q);
      if (lane == 0) L.vnorm[wave] = 1.0 / sqrt(q / (double)SH::H + c.eps);
    }
    if (tid < 32) reinterpret_cast<float*>(gh)[tid] = gr;   // gamma of this workgroup's rows (gh is free)
    __syncthreads();
    const float* gw = reinterpret_cast<const float*>(gh);
    for (int i = tid; i < nq * (nr / 2); i += BLOCK) {
      const int p = i / (nr / 2), j = 2 * (i % (nr / 2));
      const double r = L.vnorm[p];
      const float y0 = (float)(((double)L.h2res[p * 32 + j] * r) * (double)gw[j]);
      const float y1 = (float)(((double)L.h2res[p * 32 + j + 1] * r) * (double)gw[j + 1]);
      ll_put(vbuf(a, a.off.vhn, SH::H / 2, p) + (r0 + j) / 2, f32_to_bf16(y0) | (f32_to_bf16(y1) << 16), st.k1);
    }
  }
  return true;
}

// ------------------------------------------------------------------ BF: router, shared and union experts
template <class SH>
__device__ __forceinline__ bool bstage_ffn(Ctx& cx, const KArgs& a, const Step& st, VLds& L, int nq) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  const int w = cx.w, nwg = cx.nwg;
  const uint32_t k1 = st.k1;
  constexpr int H = SH::H, AST = vb_astr(H), INTER = SH::INTER;
  static_assert(SH::MOE && SH::FP8, "the batched FFN is the FP8 MoE one");
  float* tmp = reinterpret_cast<float*>(L.A + VB * AST);   // router sums, then [nq][E][2] logits, keys
  float rbias = 0.f;
  if (w < c.E && c.router == PLD_ROUTER_SIGMOID_BIAS) rbias = gp(Ly.router_bias)[w];
  const int ns = c.nshared;
  uint64_t* mbase = wsp<uint64_t>(a, a.off.vm);
  const size_t mwords = (size_t)VB * INTER / 2;   // words of one union slot
  // shared experts: this workgroup's j range, gate and up segments
  const int j0 = 2 * split_at(INTER / 2, nwg, w), j1 = 2 * split_at(INTER / 2, nwg, w + 1), nj = j1 - j0;
  __syncthreads();
  for (int s = 0; s < ns; s++) {
    const size_t bo = (size_t)(c.E + s) * Ly.gu_slot_bytes + (size_t)j0 * H;
    mseg_set(L.segs, 2 * s, Ly.w_gate.w + bo, Ly.w_gate.s + (size_t)(c.E + s) * Ly.gu_slot_scales, nj, j0, 0, 2 * s * nj, nq);
    mseg_set(L.segs, 2 * s + 1, Ly.w_up.w + bo, Ly.w_up.s + (size_t)(c.E + s) * Ly.gu_slot_scales, nj, j0, 0,
             (2 * s + 1) * nj, nq);
  }
  __syncthreads();
  auto pre = [&]() -> bool {
    const int tid = tid_opaque(), lane = tid & 63, wave = tid >> 6;
    // (1) router workgroups: expert w's logit of every position from the W_O workgroups'
    // router sums (words k < 2 nq of each producer's 16-word line, added in a fixed order:
    // lane sums in producer order, then the wave's tree) times the norm scale; published as
    // four LL words (logit lo, hi, key lo, hi) per position
    if (w < c.E) {
      struct IdxP {
        int nq2;
        __device__ __forceinline__ int operator()(int i) const { return (i / nq2) * (VB * 2) + i % nq2; }
      };
      const double* rd = reinterpret_cast<const double*>(tmp);   // [nwg][nq] (fetched fp64 pairs)
      if (!ll_fetch<per_for(256 * VB * 2)>(cx, reinterpret_cast<uint32_t*>(tmp),
                                           wsp<uint64_t>(a, a.off.vrp) + (size_t)w * nwg * VB * 2, nwg * nq * 2, k1,
                                           W_H2, IdxP{nq * 2}))
        return false;
      if (wave < nq) {
        double d = 0.0;
        for (int k = lane; k < nwg; k += 64) d += rd[k * nq + wave];
        d = wave_sum_any(d);
        const double sp = L.vnorm[wave] * d;
        if (lane < 4) {
          const double key = c.router == PLD_ROUTER_SIGMOID_BIAS ? (1.0 / (1.0 + exp_f64(-sp, L.dk))) + (double)rbias : sp;
          const uint64_t bits = (uint64_t)__double_as_longlong(lane < 2 ? sp : key);
          ll_put(vbuf(a, a.off.vlog, 4 * (size_t)c.E, wave) + 4 * w + lane, (uint32_t)(bits >> (32 * (lane & 1))), k1);
        }
      }
    }
    // (2) the FFN operand rows, normalised by their W_O workgroups (bf16 pairs)
    if (!ll_fetch_rows<H / 2>(cx, reinterpret_cast<uint32_t*>(L.A), AST / 2, vbuf(a, a.off.vhn, H / 2, 0), H / 2, nq, k1,
                              W_H2))
      return false;
    stamp(a, cx, st, TR_H2_READY);
    return true;
  };
  if (!mfma_list<H, 4>(L.segs, nj > 0 ? 2 * ns : 0, L.A, L.out, 2 * ns * nj, L.part, nq, pre)) return false;
  // shared m: silu(gate) * up as bf16 pairs, union slot s, position p
  for (int i = tid_opaque(); i < ns * nq * (nj / 2); i += BLOCK) {
    const int s = i / (nq * (nj / 2)), rem = i % (nq * (nj / 2)), p = rem / (nj / 2), jp = 2 * (rem % (nj / 2));
    const float* go = L.out + p * (2 * ns * nj) + 2 * s * nj;
    const float* uo = go + nj;
    const float m0 = silu_f(go[jp]) * uo[jp], m1 = silu_f(go[jp + 1]) * uo[jp + 1];
    ll_put(mbase + (size_t)s * mwords + (size_t)p * (INTER / 2) + (j0 + jp) / 2, f32_to_bf16(m0) | (f32_to_bf16(m1) << 16),
           k1);
  }
  stamp(a, cx, st, TR_SHARED_GEMV);
  // every position's router logits and keys in one fetch: lk[p][E][2]; wave p selects
  // position p's top-k (the same selection in every workgroup)
  double* lk = reinterpret_cast<double*>(tmp);
  if (!ll_fetch<per_for(VB * 4 * 256)>(cx, reinterpret_cast<uint32_t*>(lk), vbuf(a, a.off.vlog, 4 * (size_t)c.E, 0),
                                       nq * 4 * c.E, k1, W_RT))
    return false;
  stamp(a, cx, st, TR_RT_READY);
  if ((tid_opaque() >> 6) < nq) {
    const int lane = tid_opaque() & 63, p = tid_opaque() >> 6;
    const double* lkp = lk + (size_t)p * 2 * c.E;
    constexpr int NS = 4;   // E <= 256
    uint64_t ks[NS];
#pragma unroll
    for (int i = 0; i < NS; i++) {
      const int e = lane + 64 * i;
      const double ke = e < c.E ? lkp[2 * e + 1] : 0.0;
      const uint64_t bb = (uint64_t)__double_as_longlong(ke == 0.0 ? 0.0 : ke);
      ks[i] = e < c.E ? ((bb >> 63) ? ~bb : (bb | (1ull << 63))) : 0ull;
    }
    for (int r = 0; r < c.topk; r++) {
      uint64_t b = ks[0];
      uint32_t bi = 0u;
#pragma unroll
      for (int i = 1; i < NS; i++) {
        const bool gt = ks[i] > b;
        b = gt ? ks[i] : b;
        bi = gt ? (uint32_t)i : bi;
      }
      // wave-wide largest key with DPP moves (a lane keeps its own value where a move does
      // not write it); the result from lane 63
      uint64_t m = b;
      auto step = [&](auto ctrl_tag) {
        constexpr int CTRL = decltype(ctrl_tag)::value >> 4, RM = decltype(ctrl_tag)::value & 0xf;
        const uint64_t o = ((uint64_t)dpp_keep_u32<CTRL, RM>((uint32_t)(m >> 32)) << 32) | dpp_keep_u32<CTRL, RM>((uint32_t)m);
        m = o > m ? o : m;
      };
      step(std::integral_constant<int, (0xB1 << 4) | 0xf>{});    // quad_perm [1,0,3,2]
      step(std::integral_constant<int, (0x4E << 4) | 0xf>{});    // quad_perm [2,3,0,1]
      step(std::integral_constant<int, (0x141 << 4) | 0xf>{});   // row_half_mirror
      step(std::integral_constant<int, (0x140 << 4) | 0xf>{});   // row_mirror
      step(std::integral_constant<int, (0x142 << 4) | 0xa>{});   // row_bcast:15
      step(std::integral_constant<int, (0x143 << 4) | 0xc>{});   // row_bcast:31
      m = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(m >> 32), 63) << 32) |
          (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)m, 63);
      const uint32_t mye = (uint32_t)lane + 64u * bi;
      const bool hold = b == m;
      const uint64_t hm = __ballot(hold);
      const uint32_t ee = __popcll(hm) == 1
                              ? (uint32_t)__builtin_amdgcn_readlane((int)mye, __ffsll((unsigned long long)hm) - 1)
                              : wave_minmax_u32<false>(hold ? mye : 0xffffffffu);
#pragma unroll
      for (int i = 0; i < NS; i++) ks[i] = (mye == ee && bi == (uint32_t)i) ? 0ull : ks[i];
      if (lane == 0) L.isel[p * 8 + r] = (int)ee;
    }
  }
  __syncthreads();
  {
    // gates of (position p, rank r): softmax over the position's selected logits, or their
    // sigmoid scores normalised over the selection
    const bool sig = c.router == PLD_ROUTER_SIGMOID_BIAS;
    double* num = lk + (size_t)VB * 2 * 256;   // [VB][8]
    const int t = tid_opaque(), p = t / 8, r = t % 8;
    if (p < nq && r < c.topk) {
      const double* lkp = lk + (size_t)p * 2 * c.E;
      const double x = lkp[2 * L.isel[p * 8 + r]];
      num[t] = sig ? 1.0 / (1.0 + exp_f64(-x, L.dk)) : exp_f64(x - lkp[2 * L.isel[p * 8]], L.dk);
    }
    __syncthreads();
    if (p < nq && r < c.topk) {
      double gsum = 0.0;
      for (int j = 0; j < c.topk; j++) gsum += num[p * 8 + j];
      L.fgate[p * 8 + r] = (float)(num[t] / gsum);
    }
    __syncthreads();
  }
  stamp(a, cx, st, TR_TOPK);
  // union of the selected experts, ascending, slots after the shared ones: thread (p, r) sets
  // bit p of its expert's mask (LDS atomic OR: the result does not depend on the order),
  // then thread e places expert e by a ballot count over the lower experts
  {
    static_assert(BLOCK >= 256, "one thread per expert");
    int* flag = reinterpret_cast<int*>(tmp);   // [E] position masks
    int* wcnt = flag + 256;                     // [NWAVES] experts in use per wave
    const int tid = tid_opaque(), lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < c.E; e += BLOCK) flag[e] = 0;
    __syncthreads();
    if (tid < nq * 8 && (tid & 7) < c.topk) atomicOr(&flag[L.isel[tid]], 1 << (tid >> 3));
    __syncthreads();
    const int fe = tid < c.E ? flag[tid] : 0;
    const uint64_t on = __ballot(fe != 0);
    if (lane == 0) wcnt[wave] = __popcll(on);
    __syncthreads();
    int off = 0;
    for (int v = 0; v < wave; v++) off += wcnt[v];
    if (fe != 0) {
      const int u = off + __popcll(on & ((1ull << lane) - 1ull));
      L.uexp[ns + u] = tid;
      L.umask[ns + u] = fe;
    }
    if (tid < ns) {
      L.uexp[tid] = c.E + tid;
      L.umask[tid] = (1 << nq) - 1;
    }
    if (tid == 0) {
      int tot = 0;
      for (int v = 0; v < NWAVES; v++) tot += wcnt[v];
      L.misc[0] = ns + tot;
    }
    __syncthreads();
  }
  if (w == 0 && tid_opaque() < nq * c.topk) {
    const int p = tid_opaque() / c.topk, r = tid_opaque() % c.topk;
    st_u32(reinterpret_cast<uint32_t*>(wsp<int>(a, a.off.vsel)) + p * 8 + r, (uint32_t)L.isel[p * 8 + r]);
    st_f32(wsp<float>(a, a.off.vsel) + VB * 8 + p * 8 + r, L.fgate[p * 8 + r]);
  }
  // routed union slots: this workgroup's share of the (slot, row) pairs, in pairs of rows
  const int nu = L.misc[0] - ns;
  const int tot = nu * INTER;
  const int i0 = 2 * split_at(tot / 2, nwg, w), i1 = 2 * split_at(tot / 2, nwg, w + 1);
  // (pieces kept in LDS: a per-lane array indexed at run time would live in scratch memory)
  int npc = 0;
  int* pu = L.pcs;
  int* pj0 = L.pcs + MAX_MSEGS / 2;
  int* pj1 = L.pcs + MAX_MSEGS;
  __syncthreads();
  for (int u = i0 / INTER; u < nu && u * INTER < i1 && npc < MAX_MSEGS / 2; u++) {
    const int lo = max(i0, u * INTER) - u * INTER, hi = min(i1, (u + 1) * INTER) - u * INTER;
    if (lo < hi) {
      if (tid_opaque() == 0) {
        pu[npc] = u; pj0[npc] = lo; pj1[npc] = hi;
      }
      npc++;
    }
  }
  __syncthreads();
  int nrows = 0;
  for (int q = 0; q < npc; q++) nrows += 2 * (pj1[q] - pj0[q]);
  {
    int oo = 0;
    for (int q = 0; q < npc; q++) {
      const int e = L.uexp[ns + pu[q]], nn = pj1[q] - pj0[q];
      const size_t bo = (size_t)e * Ly.gu_slot_bytes + (size_t)pj0[q] * H;
      mseg_set(L.segs, 2 * q, Ly.w_gate.w + bo, Ly.w_gate.s + (size_t)e * Ly.gu_slot_scales, nn, pj0[q], 0, oo, nq);
      mseg_set(L.segs, 2 * q + 1, Ly.w_up.w + bo, Ly.w_up.s + (size_t)e * Ly.gu_slot_scales, nn, pj0[q], 0, oo + nn, nq);
      oo += 2 * nn;
    }
  }
  __syncthreads();
  float* rout = tmp;   // [nq][nrows] (the router scratch is free now)
  if (!mfma_list<H, 4>(L.segs, 2 * npc, L.A, rout, nrows, L.part, nq, NoPre{})) return false;
  {
    int oo = 0;
    for (int q = 0; q < npc; q++) {
      const int nn = pj1[q] - pj0[q], u = pu[q], msk = L.umask[ns + u];
      for (int i = tid_opaque(); i < nq * (nn / 2); i += BLOCK) {
        const int p = i / (nn / 2), jp = 2 * (i % (nn / 2));
        if (!((msk >> p) & 1)) continue;
        const float* go = rout + p * nrows + oo;
        const float* uo = go + nn;
        const float m0 = silu_f(go[jp]) * uo[jp], m1 = silu_f(go[jp + 1]) * uo[jp + 1];
        ll_put(mbase + (size_t)(ns + u) * mwords + (size_t)p * (INTER / 2) + (pj0[q] + jp) / 2,
               f32_to_bf16(m0) | (f32_to_bf16(m1) << 16), k1);
      }
      oo += 2 * nn;
    }
  }
  stamp(a, cx, st, TR_M_STORED);
  return true;
}

// ------------------------------------------------------------------ BD: down projections of every (slot, position)
// Work items are (union slot, 16-row tile of the output) pairs, slot-major, split evenly over
// the workgroups: a workgroup streams whole tiles of one or two slots' down matrices and
// fetches only those slots' activation vectors. Each tile's results, times the position's
// gate, go out as LL words (fpart[slot][position][row]); then the workgroup that owns output
// rows [r0, r1) adds, per position, its slots' partials in a fixed order (shared experts,
// then the position's experts in rank order) and the residual.
template <class SH>
__device__ __forceinline__ bool bstage_down(Ctx& cx, const KArgs& a, const Step& st, VLds& L, int nq, bool last_layer,
                                            uint16_t* out_hidden) {
  const KCfg& c = a.c;
  const DLayer Ly = *gp(st.Ly);
  constexpr int H = SH::H, INTER = SH::INTER, AST = vb_astr(INTER), NT = H / 16;
  static_assert(H % 16 == 0, "whole tiles");
  const int w = cx.w, nwg = cx.nwg;
  const int ns = c.nshared, nslot = L.misc[0];
  uint64_t* mbase = wsp<uint64_t>(a, a.off.vm);
  uint64_t* fpart = wsp<uint64_t>(a, a.off.vfp);
  const int mwords = VB * INTER / 2;
  // this workgroup's (slot, tile) items [i0, i1): one segment per slot run
  const int tot = nslot * NT;
  const int i0 = split_at(tot, nwg, w), i1 = split_at(tot, nwg, w + 1);
  __syncthreads();
  int nseg = 0, nv = 0, nrows = 0;
  for (int s = i0 / NT; s < nslot && s * NT < i1; s++) {
    const int t0 = max(i0, s * NT) - s * NT, t1 = min(i1, (s + 1) * NT) - s * NT;
    if (t0 >= t1) continue;
    const int e = L.uexp[s], msk = L.umask[s];
    if (tid_opaque() == 0) {
      MSeg& S = L.segs[nseg];
      S.w = Ly.w_down.w + (size_t)e * Ly.dn_slot_bytes + (size_t)t0 * 16 * INTER;
      S.s = Ly.w_down.s + (size_t)e * Ly.dn_slot_scales;
      S.n = (t1 - t0) * 16;
      S.srow = t0 * 16;
      S.a_off = 0;
      S.o_off = nrows * VB;
      int v = nv;
      for (int p = 0; p < VB; p++) {
        const bool on = p < nq && ((msk >> p) & 1);
        S.vrow[p] = (int8_t)(on ? v : -1);
        if (on) L.vsrc[v++] = s * mwords + p * (INTER / 2);
      }
      L.pcs[nseg] = s;   // the slot of segment nseg
    }
    nv += __popc(msk & ((1 << nq) - 1));
    nrows += (t1 - t0) * 16;
    nseg++;
  }
  __syncthreads();
  // at most two slots per workgroup (items per workgroup <= tiles per slot): <= 2 * VB vectors
  float* res = reinterpret_cast<float*>(L.A + 2 * VB * AST);   // segment g's results at (o_off + p * rows_g + r)
  auto pre = [&]() -> bool {
    struct IdxV {
      const int* vs;
      __device__ __forceinline__ int operator()(int i) const { return vs[i / (INTER / 2)] + i % (INTER / 2); }
    };
    if (!ll_fetch<per_for(32 * INTER / 2)>(cx, reinterpret_cast<uint32_t*>(L.A), mbase, nv * (INTER / 2), st.k1, W_M,
                                           IdxV{L.vsrc}, StRows<INTER / 2>{AST / 2}))
      return false;
    stamp(a, cx, st, TR_M_READY);
    return true;
  };
  // (ostr 0: segment g's results form a [VB][rows_g] block at o_off = rows before g * VB)
  if (!mfma_list<INTER, 4>(L.segs, nseg, L.A, res, 0, L.part, nq, pre)) return false;
  stamp(a, cx, st, TR_DOWN_GEMV);
  // gated partials out: fpart[slot][p][row]
  {
    int ob = 0;
    for (int g = 0; g < nseg; g++) {
      const MSeg& S = L.segs[g];
      const int sl = L.pcs[g], e = L.uexp[sl];
      for (int i = tid_opaque(); i < nq * S.n; i += BLOCK) {
        const int p = i / S.n, r = i % S.n;
        if (S.vrow[p] < 0) continue;
        float gte = 1.f;
        if (sl >= ns) {
          gte = 0.f;
          for (int k = 0; k < c.topk; k++)
            if (L.isel[p * 8 + k] == e) gte = L.fgate[p * 8 + k];
        }
        ll_put_f32(fpart + ((size_t)sl * VB + p) * H + S.srow + r, gte * res[ob * VB + p * S.n + r], st.k1);
      }
      ob += S.n;
    }
  }
  // the union slot of each position's experts (rank order), for the reduction
  if (tid_opaque() < nq * c.topk) {
    const int p = tid_opaque() / c.topk, k = tid_opaque() % c.topk, e = L.isel[p * 8 + k];
    int sl = ns;
    while (L.uexp[sl] != e) sl++;
    L.vslot[p * 8 + k] = sl;
  }
  __syncthreads();
  // reduction of the rows [r0, r1) this workgroup owns: per position ns + topk partials
  int r0, r1;
  hrows(H, nwg, w, &r0, &r1);
  const int nr = r1 - r0, per = (ns + c.topk) * nr;
  struct IdxF {
    const int* vslot;
    int per, nr, ns, topk, r0;
    __device__ __forceinline__ int operator()(int i) const {
      const int p = i / per, k = (i % per) / nr, r = i % nr;
      const int sl = k < ns ? k : vslot[p * 8 + (k - ns)];
      return (sl * VB + p) * SH::H + r0 + r;
    }
  };
  float* fr = reinterpret_cast<float*>(L.A);   // [nq][ns + topk][nr]
  if (!ll_fetch<per_for(VB * 10 * 32)>(cx, reinterpret_cast<uint32_t*>(fr), fpart, nq * per, st.k1, W_M,
                                       IdxF{L.vslot, per, nr, ns, c.topk, r0}))
    return false;
  for (int i = tid_opaque(); i < nq * (nr / 2); i += BLOCK) {
    const int p = i / (nr / 2), r = 2 * (i % (nr / 2));
    float f0 = 0.f, f1 = 0.f;
    for (int k = 0; k < ns + c.topk; k++) {
      f0 += fr[p * per + k * nr + r];
      f1 += fr[p * per + k * nr + r + 1];
    }
    st_f32(wsp<float>(a, a.off.vf) + (size_t)p * H + r0 + r, f0);   // debug copy of f
    st_f32(wsp<float>(a, a.off.vf) + (size_t)p * H + r0 + r + 1, f1);
    const uint32_t lo = f32_to_bf16(L.h2res[p * 32 + r] + f0);
    const uint32_t hi = f32_to_bf16(L.h2res[p * 32 + r + 1] + f1);
    ll_put(vbuf(a, a.off.vx, H / 2, p) + (r0 + r) / 2, lo | (hi << 16), st.k1);
    if (last_layer && out_hidden && p == nq - 1) gp(reinterpret_cast<uint32_t*>(out_hidden))[(r0 + r) / 2] = lo | (hi << 16);
  }
  stamp(a, cx, st, TR_DOWN_DONE);
  return true;
}

// ------------------------------------------------------------------ the batched kernel
// Verify (BM == 0): a.nrows positions from a.pos0 of one sequence; position 0 takes
// a.in_token, position p > 0 the caller's draft p - 1 (clamped into the vocabulary).
// Per-position logits and tokens, and the count of leading drafts equal to the token
// chosen at the position before.
// Batch decode (BM == 1): a.nrows sequences, row p at cache position a.bpos[p] of its
// own cache, fed a.btok[p]; a.n_tokens steps, each choosing every row's next token, which
// is the row's input at the next step.
static_assert(VB == 8, "KArgs holds 8 rows of batch positions and tokens");
// The two modes are separate instantiations (a.bmode == BM), so each compiles only its own
// attention stage and neither's register allocation depends on the other's.
template <class SH, int BM>
__global__ void __launch_bounds__(BLOCK, 1) k_verify_mla(KArgs a) {
  extern __shared__ float lds_raw[];
  Ctx cx;
  cx.budget = a.budget;
  cx.w = blockIdx.x;
  cx.nwg = gridDim.x;
  cx.status = wsp<uint32_t>(a, a.off.status);
  cx.wacc = nullptr;
  const DLayer* layers = wsp<DLayer>(a, a.off.layers);
  if ((a.hooks & PLD_HOOK_DROP_WG0) && cx.w == 0) return;
  const int nq = a.nrows;
  const int nsteps = BM ? a.n_tokens : 1;
  VLds L = vcarve(lds_raw);
  if (tid_opaque() < TR_SLOTS) L.tr[tid_opaque()] = 0;
  exp_f64_init(L.dk);
  __syncthreads();
  if (tid_opaque() < nq) {
    const int p = tid_opaque();
    if (BM) {
      L.tok[p] = a.btok[p];
      L.rpos[p] = a.bpos[p];
    } else {
      L.tok[p] = p == 0 ? a.in_token : min(max(gp(a.drafts)[p - 1], 0), a.c.vocab - 1);
      L.rpos[p] = a.pos0 + p;
    }
  }
  __syncthreads();
  Lds HL = head_lds(L);
  for (int t = 0; t < nsteps; t++) {
    for (int li = 0; li < a.n_layers; li++) {
      cx.layer = a.layer0 + li;
      cx.token = t;
      Step st;
      st.Ly = layers + a.layer0 + li;
      st.idx = t * a.n_layers + li;
      st.k1 = a.step0 + (uint32_t)st.idx + 1u;
      st.first = false;
      st.in_hidden = nullptr;
      st.pos = a.pos0;
      st.emb_row = nullptr;
      st.tr = L.tr;
      KArgs as = a;
      as.bmode = BM;   // (a constant for the stages)
      asm volatile("" : "+s"(as.ws));
      Ctx cs = cx;
      asm volatile("" : "+s"(cs.w), "+s"(cs.nwg), "+s"(as.c.cpw), "+s"(as.c.cpg));
      cs.wacc = (a.trace && st.idx < a.trace_steps) ? L.tr + TR_WAIT : nullptr;
      stamp(as, cs, st, TR_START);
      if (!bstage_x<SH>(cs, as, st, L, nq, li)) return;
      if (!bstage_q<SH>(cs, as, st, L, nq)) return;
      if (!bstage_absorb<SH>(cs, as, st, L, nq)) return;
      if (BM == 0) {
        if (!bstage_attn_v<SH>(cs, as, st, L, nq)) return;
      } else {
        if (!bstage_attn<SH>(cs, as, st, L, nq)) return;
      }
      if (!bstage_merge<SH>(cs, as, st, L, nq)) return;
      if (!bstage_uv<SH>(cs, as, st, L, nq)) return;
      if (!bstage_wo<SH>(cs, as, st, L, nq)) return;
      if (!bstage_ffn<SH>(cs, as, st, L, nq)) return;
      if (!bstage_down<SH>(cs, as, st, L, nq, t == nsteps - 1 && li == a.n_layers - 1, as.out_hidden)) return;
      trace_flush(as, cs, st);
    }
    // LM head and token choice of every row (the single-position head stage, on each row's
    // final hidden state; its candidate words in a buffer of the row's own)
    const uint32_t kl = a.step0 + (uint32_t)((t + 1) * a.n_layers);
    for (int p = 0; p < nq; p++) {
      KArgs ah = a;
      ah.off.x = a.off.vx + (size_t)p * (SH::H / 2) * 8;
      ah.off.amax = a.off.vamax + (size_t)p * 3 * cx.nwg * 8;
      Step st;
      st.Ly = layers + a.layer0 + a.n_layers - 1;
      st.idx = (t + 1) * a.n_layers;
      st.k1 = kl;
      st.first = false;
      st.in_hidden = nullptr;
      st.pos = L.rpos[p];
      st.emb_row = nullptr;
      st.tr = L.tr;
      cx.token = t;
      int tk = 0;
      if (!stage_head<SH>(cx, ah, st, HL, t * nq + p, &tk)) return;
      if (tid_opaque() == 0) L.tok[VB + p] = tk;
    }
    __syncthreads();
    if (BM && tid_opaque() < nq) {   // each row's chosen token is its next input
      L.tok[tid_opaque()] = L.tok[VB + tid_opaque()];
      L.rpos[tid_opaque()] += 1;
    }
    __syncthreads();
  }
  if (!BM && cx.w == 0 && tid_opaque() == 0 && a.out_accepted) {
    int acc = 0;
    for (int p = 1; p < nq; p++) {
      if (gp(a.drafts)[p - 1] != L.tok[VB + p - 1]) break;
      acc++;
    }
    gp(a.out_accepted)[0] = acc;
  }
}
