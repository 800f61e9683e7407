// Device building blocks of the persistent decode kernel (gfx950, wave64).
//
// Synchronisation protocol (measured on MI355X before it was chosen):
//  * Cross-workgroup data (activations, attention partials, appended cache rows) is
//    written with agent-scope relaxed atomic stores, which write through to the
//    device coherence point, and read back with agent-scope relaxed atomic loads.
//    No L2 write-back or invalidate is needed per stage; weights use ordinary
//    (non-temporal) loads because they are never written.
//  * Activations move as LL words: each 8-byte store holds a 32-bit payload and the
//    step's epoch, so the consumer polls the data itself. A handoff then costs about
//    one store plus one load round trip; a counter barrier (drain the stores, count
//    per XCD, count globally, poll) cost four to five, i.e. ~10 us per stage boundary
//    while HBM is busy, because every round trip queues behind the weight stream.
//  * Only static weights may be loaded before an activation is read. This is the
//    ordering rule the vLLM Kimi K3 backend article reports from its kernel audit
//    (section "Agent-written kernels face evidence gates").
//  * A wave's loads return in order, so a latency-critical load waits for every weight
//    load the wave issued before it: prefetch depth is kept to what HBM needs.
//  * Every wait is bounded by a wall-clock deadline; on expiry the workgroup records
//    a status word, raises a global abort flag and leaves, and so do all others.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pld {

constexpr int BLOCK = 512;
constexpr int NWAVES = BLOCK / 64;
constexpr int NXCD = 8;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// (the attribute only exists for the device pass; hipcc's host pass parses the same code)
#if defined(__HIP_DEVICE_COMPILE__)
#define PLD_GLOBAL __attribute__((address_space(1)))
#else
#define PLD_GLOBAL
#endif

// Every pointer handed to the kernel addresses device (global) memory; saying so lets
// the compiler emit global_* instead of flat_* instructions (flat accesses also count
// against the LDS counter, which would make a wait on LDS drain the weight prefetch).
template <typename T>
__device__ __forceinline__ PLD_GLOBAL T* gp(T* p) { return (PLD_GLOBAL T*)(p); }
template <typename T>
__device__ __forceinline__ const PLD_GLOBAL T* gp(const T* p) { return (const PLD_GLOBAL T*)(p); }
// The same for LDS (atomics then compile to ds_* instead of flat_* instructions).
#if defined(__HIP_DEVICE_COMPILE__)
#define PLD_LDS __attribute__((address_space(3)))
#else
#define PLD_LDS
#endif
template <typename T>
__device__ __forceinline__ PLD_LDS T* lds_ptr(T* p) { return (PLD_LDS T*)(p); }

// tid_opaque() as a value the compiler cannot treat as loop-invariant: per-lane addresses
// computed from it inside a helper are then not hoisted out of the layer loop, where they
// would stay live (and spill) across every stage.
__device__ __forceinline__ int tid_opaque() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// 16-byte streaming load of static weights (non-temporal hint: read once per step)
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load((const PLD_GLOBAL u32x4*)(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld_g16(const void* p) {
  const u32x4 v = *(const PLD_GLOBAL u32x4*)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ----------------------------------------------------------------- memory helpers
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_u32(const uint32_t* p) {
  return __hip_atomic_load(gp(const_cast<uint32_t*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_f32(float* p, float v) { st_u32(reinterpret_cast<uint32_t*>(p), __float_as_uint(v)); }
__device__ __forceinline__ float ld_f32(const float* p) { return __uint_as_float(ld_u32(reinterpret_cast<const uint32_t*>(p))); }
__device__ __forceinline__ uint64_t ld_u64(const uint64_t* p) {
  return __hip_atomic_load(gp(const_cast<uint64_t*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The same loads/stores addressed as uniform base + 32-bit byte offset: the compiler can
// use the scalar-base + 32-bit vector-offset form, so no 64-bit per-lane address has to
// stay live across the layer loop.
__device__ __forceinline__ uint64_t ld_u64_off(const void* base, uint32_t byte_off) {
  const PLD_GLOBAL char* b = gp(reinterpret_cast<const char*>(base));
  return __hip_atomic_load((PLD_GLOBAL uint64_t*)(b + byte_off), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_u32_off(const void* base, uint32_t byte_off) {
  const PLD_GLOBAL char* b = gp(reinterpret_cast<const char*>(base));
  return __hip_atomic_load((PLD_GLOBAL uint32_t*)(b + byte_off), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------- number formats
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
// fp64 -> bf16, round to nearest even in ONE rounding (going through fp32 would round
// twice): the 45 low mantissa bits are rounded away on the fp64 bit pattern, after
// which the value has 8 significant bits and converts to fp32 exactly. Finite values in
// the fp32 normal range.
__device__ __forceinline__ uint32_t f64_to_bf16(double x) {
  uint64_t b = (uint64_t)__double_as_longlong(x);
  b += 0x00000FFFFFFFFFFFull + ((b >> 45) & 1ull);
  b &= ~0x00001FFFFFFFFFFFull;
  return __float_as_uint((float)__longlong_as_double((long long)b)) >> 16;
}
// fp32 -> OCP E4M3FN code, round to nearest with ties to the even code, for |q| <= 448
// (no saturation or NaN handling needed in that range). Normal codes keep 3 mantissa
// bits of q's fp32 significand; below 2^-6 the grid is the subnormal step 2^-9, reached
// from the 24-bit significand by a right shift of 14 - e. A value that rounds up to the
// next binade lands on its code because code = (biased exponent << 3) + mantissa is
// continuous. The sign bit is kept for values that round to zero.
__device__ __forceinline__ uint32_t e4m3_encode(float q) {
  const uint32_t u = __float_as_uint(q);
  const uint32_t sgn = (u >> 24) & 0x80u;
  const uint32_t mag = u & 0x7fffffffu;
  const int e = (int)(mag >> 23) - 127;
  const uint32_t full = (mag & 0x7fffffu) | 0x800000u;
  uint32_t code;
  if (e >= -6) {
    uint32_t q3 = (mag >> 20) & 7u;
    const uint32_t rem = mag & 0xfffffu;
    q3 += (rem > 0x80000u || (rem == 0x80000u && (q3 & 1u))) ? 1u : 0u;
    code = ((uint32_t)(e + 7) << 3) + q3;
  } else if (e >= -10) {
    const int sh = 14 - e;   // 21 .. 24
    uint32_t qq = full >> sh;
    const uint32_t rem = full & ((1u << sh) - 1u), half = 1u << (sh - 1);
    qq += (rem > half || (rem == half && (qq & 1u))) ? 1u : 0u;
    code = qq;
  } else {
    code = 0u;   // below half of the smallest subnormal step (fp32 zero and denormals included)
  }
  return sgn | code;
}

// ----------------------------------------------------------------- reductions
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
  return v;
}
// Sum over groups of N consecutive lanes (N = 8, 16, 32 or 64) with DPP lane moves, which
// run in the vector ALU (a __shfl_xor compiles to an LDS permute). The group sum is valid
// in the group's LAST lane (for N = 8 and 16 in every lane of the group).
template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, BOUND));
}
template <int N>
__device__ __forceinline__ float dpp_sum(float v) {
  static_assert(N == 8 || N == 16 || N == 32 || N == 64, "group size");
  v += dpp_mov<0xB1, 0xf, false>(v);    // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E, 0xf, false>(v);    // quad_perm [2,3,0,1]
  v += dpp_mov<0x141, 0xf, false>(v);   // row_half_mirror: sums of 8
  if constexpr (N >= 16) v += dpp_mov<0x140, 0xf, false>(v);   // row_mirror: sums of 16 (each row)
  // row_bcast15: lane 15 of row r is added into row r+1 (only rows 1 and 3 are written)
  if constexpr (N >= 32) v += dpp_mov<0x142, 0xa, true>(v);
  // row_bcast31: lane 31 is added into rows 2 and 3
  if constexpr (N >= 64) v += dpp_mov<0x143, 0xc, true>(v);
  return v;
}

// 32-bit integer DPP move (bound_ctrl: lanes whose source is out of range read 0).
template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xf, BOUND);
}
// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele inside each row of 16
// (row_shr 1, 2, 4, 8), then row 0's total into row 1 and row 2's into row 3 (row_bcast15),
// then the total of rows 0-1 into rows 2 and 3 (row_bcast31).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  x += dpp_u32<0x111, 0xf, true>(x);
  x += dpp_u32<0x112, 0xf, true>(x);
  x += dpp_u32<0x114, 0xf, true>(x);
  x += dpp_u32<0x118, 0xf, true>(x);
  x += dpp_u32<0x142, 0xa, true>(x);
  x += dpp_u32<0x143, 0xc, true>(x);
  return x;
}
// Wave-wide min / max of u32 with DPP moves (a lane keeps its own value where a move does
// not write it); the result, from lane 63, in every lane.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_keep_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, ROW_MASK, 0xf, false);
}
template <bool MAX>
__device__ __forceinline__ uint32_t wave_minmax_u32(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
  v = op(v, dpp_keep_u32<0xB1, 0xf>(v));
  v = op(v, dpp_keep_u32<0x4E, 0xf>(v));
  v = op(v, dpp_keep_u32<0x141, 0xf>(v));
  v = op(v, dpp_keep_u32<0x140, 0xf>(v));
  v = op(v, dpp_keep_u32<0x142, 0xa>(v));
  v = op(v, dpp_keep_u32<0x143, 0xc>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// Sum over each row of 16 lanes, valid in every lane of the row.
__device__ __forceinline__ uint32_t row16_sum_u32(uint32_t x) {
  x += dpp_u32<0xB1, 0xf, false>(x);
  x += dpp_u32<0x4E, 0xf, false>(x);
  x += dpp_u32<0x141, 0xf, false>(x);
  x += dpp_u32<0x140, 0xf, false>(x);
  return x;
}

// Wave-wide sum of u32: row sums, then rows 0+1 and 2+3 (row_bcast15), then all four
// (row_bcast31, valid in rows 2-3); the result, from lane 63, in every lane.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  x = row16_sum_u32(x);
  x += dpp_u32<0x142, 0xa, true>(x);
  x += dpp_u32<0x143, 0xc, true>(x);
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// fp64 sum over groups of 64 lanes with DPP moves applied to both 32-bit halves (same
// move sequence as dpp_sum<64>); the total is valid in lane 63.
template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ double dpp_mov_f64(double x) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xffffffff), CTRL, ROW_MASK, 0xf, BOUND);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, ROW_MASK, 0xf, BOUND);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
template <int N>
__device__ __forceinline__ double dpp_sum_f64(double v) {
  static_assert(N == 8 || N == 16 || N == 32 || N == 64, "group size");
  v += dpp_mov_f64<0xB1, 0xf, false>(v);
  v += dpp_mov_f64<0x4E, 0xf, false>(v);
  v += dpp_mov_f64<0x141, 0xf, false>(v);
  if constexpr (N >= 16) v += dpp_mov_f64<0x140, 0xf, false>(v);
  if constexpr (N >= 32) v += dpp_mov_f64<0x142, 0xa, true>(v);
  if constexpr (N >= 64) v += dpp_mov_f64<0x143, 0xc, true>(v);
  return v;
}
__device__ __forceinline__ double dpp_sum64_f64(double v) { return dpp_sum_f64<64>(v); }

// Wave-wide max and sum with DPP lane moves (no LDS permutes), result in every lane.
// The moves keep a lane's own value where a move does not write it (old = the value,
// bound_ctrl off), so max is not polluted by zeros; same move sequence as dpp_sum.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_keep(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_keep<0xB1, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x4E, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x141, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x140, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x142, 0xa>(v));
  v = fmaxf(v, dpp_keep<0x143, 0xc>(v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Max and sum over each 32-lane half of a wave with DPP moves: row results in every lane,
// then rows 0+1 and 2+3 (row_bcast15); each lane gets its half's result (lanes 31, 63).
__device__ __forceinline__ float half_max_dpp(float v) {
  v = fmaxf(v, dpp_keep<0xB1, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x4E, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x141, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x140, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x142, 0xa>(v));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  return (tid_opaque() & 32) ? b : a;
}
__device__ __forceinline__ float half_sum_dpp(float v) {
  v += dpp_mov<0xB1, 0xf, false>(v);
  v += dpp_mov<0x4E, 0xf, false>(v);
  v += dpp_mov<0x141, 0xf, false>(v);
  v += dpp_mov<0x140, 0xf, false>(v);
  v += dpp_mov<0x142, 0xa, true>(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  return (tid_opaque() & 32) ? b : a;
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = dpp_sum<64>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Wave sums with DPP moves (no LDS permutes); the result, from lane 63, in every lane.
__device__ __forceinline__ float wave_sum_any(float v) { return wave_sum_dpp(v); }
__device__ __forceinline__ double wave_sum_any(double v) {
  v = dpp_sum64_f64(v);
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffff), 63);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), 63);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Block-wide sum in a fixed order (wave sums, then wave 0..7 in order). All threads get the result.
template <typename T>
__device__ __forceinline__ T block_sum(T v, T* red) {
  v = wave_sum_any(v);
  const int lane = tid_opaque() & 63, wave = tid_opaque() >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  T s = 0;
#pragma unroll
  for (int i = 0; i < NWAVES; i++) s += red[i];
  __syncthreads();
  return s;
}

// ----------------------------------------------------------------- dot products
// 8 bf16 weights (one 16-byte chunk) against 8 fp32 activations
__device__ __forceinline__ float dot8_bf16(const uint4& v, const float* a) {
  float s = 0.f;
  s = fmaf(bf_lo(v.x), a[0], s); s = fmaf(bf_hi(v.x), a[1], s);
  s = fmaf(bf_lo(v.y), a[2], s); s = fmaf(bf_hi(v.y), a[3], s);
  s = fmaf(bf_lo(v.z), a[4], s); s = fmaf(bf_hi(v.z), a[5], s);
  s = fmaf(bf_lo(v.w), a[6], s); s = fmaf(bf_hi(v.w), a[7], s);
  return s;
}
// the same in fp64 (bf16 x fp32 products are exact in fp64)
__device__ __forceinline__ double dot8_bf16_f64(const uint4& v, const float* a) {
  double s = 0.0;
  s = fma((double)bf_lo(v.x), (double)a[0], s); s = fma((double)bf_hi(v.x), (double)a[1], s);
  s = fma((double)bf_lo(v.y), (double)a[2], s); s = fma((double)bf_hi(v.y), (double)a[3], s);
  s = fma((double)bf_lo(v.z), (double)a[4], s); s = fma((double)bf_hi(v.z), (double)a[5], s);
  s = fma((double)bf_lo(v.w), (double)a[6], s); s = fma((double)bf_hi(v.w), (double)a[7], s);
  return s;
}
// 16 OCP E4M3FN weights against 16 fp32 activations (hardware fp8 -> fp32 conversion)
__device__ __forceinline__ float dot16_fp8(const uint4& v, const float* a) {
  float s = 0.f;
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)d[i], false);
    f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)d[i], true);
    s = fmaf(lo.x, a[4 * i + 0], s);
    s = fmaf(lo.y, a[4 * i + 1], s);
    s = fmaf(hi.x, a[4 * i + 2], s);
    s = fmaf(hi.y, a[4 * i + 3], s);
  }
  return s;
}

// ----------------------------------------------------------------- weight matrices
struct DMat {
  const uint8_t* w;    // [rows][cols] bf16 or fp8 bytes
  const float* s;      // FP8 scales [ceil(rows/128)][sbk]
  int rows, cols, sbk; // sbk = ceil(cols/128)
};

// Output handling of a GEMV: out[r - r0] = v (store) or out[r - r0] += alpha * v.
enum OutMode { OUT_STORE = 0, OUT_ACCUM = 1 };

// Activation vectors that an FP8 gemv_list reads are stored padded in LDS: element e at
// float e + 4 * (e / 64). A lane reads its 16 consecutive elements (64 bytes) as float4s;
// unpadded, the spans of 16 neighbouring lanes start on only four distinct 4-bank groups
// of the 64 banks, a 4-way conflict on every activation read (measured: 186 M conflict
// cycles per 8-layer step of the FP8 MLA layer, 21 M padded). With four spare floats after
// every 64 they start on 16 distinct groups. A 16-element chunk never crosses a 64-element
// block, so it stays contiguous. Vectors of length n take apad<true>(n) floats (n a
// multiple of 64). bf16 GEMVs (32-byte spans) measured no conflicts unpadded and keep the
// plain layout (PAD = false: the identity).
template <bool PAD>
__host__ __device__ constexpr int apad(int e) { return PAD ? e + ((e >> 6) << 2) : e; }

// Lane layout per reduction length K (elements) and weight format, fixed at compile time:
// LPR lanes per row, CPL 16-byte chunks per lane and row, U rows in flight per wave
// (U*CPL ~ INFL loads of 16 bytes per lane: INFL * 8 KB in flight per 512-thread workgroup).
template <bool FP8, int K, int INFL>
struct GemvLayout {
  static constexpr int EPC = FP8 ? 16 : 8;
  static constexpr int CHUNKS = K / EPC;
  // lanes per row: the largest of 64 / 32 / 16 that divides the row's chunk count
  static constexpr int LPR = CHUNKS % 64 == 0 ? 64 : CHUNKS % 32 == 0 ? 32 : CHUNKS % 16 == 0 ? 16 : CHUNKS;
  static constexpr int CPL = CHUNKS / LPR;
  static constexpr int U0 = INFL / CPL;
  static constexpr int U = U0 < 1 ? 1 : (U0 > 12 ? 12 : U0);
  static_assert(K % EPC == 0 && CHUNKS % LPR == 0 && (LPR == 16 || LPR == 32 || LPR == 64), "unsupported K");
};

// A GEMV task is a list of row segments streamed as one pipeline: segment s holds n
// consecutive rows starting at w (row stride K elements), FP8 scales s (row-block
// stride ceil(K/128)) with row offset srow, reads the activation at act + act_off, and
// scales its row results by alpha (OUT_ACCUM). Results land in out[] in list order.
// Activations are in the layout apad<FP8>, and act_off is an offset in that layout (the
// apad of a multiple of 64 elements).
struct RowSeg {
  const uint8_t* w;
  const float* s;
  int n;
  int srow;      // row index of w's first row inside its scale grid (FP8)
  int act_off;
  float alpha;
};
constexpr int MAX_SEGS = 12;

// Streams the rows of a segment list against fp32 activation vectors in LDS.
//  * LPR lanes share one row (64/LPR rows per wave pass); each lane reads CPL 16-byte
//    chunks per row, chunk j of lane l covering elements [(j*LPR + l) * EPC, +EPC);
//  * a wave keeps U rows of loads in flight; the pipeline runs through all segments;
//  * the first U rows are issued BEFORE `pre()` runs -- pre is where the caller waits
//    for its dependency and stages the activation into LDS -- so the wait overlaps with
//    the first weight bytes arriving; only static weights are loaded ahead of a wait;
//  * partial sums are reduced across the LPR lanes and the row's first lane writes the
//    result into out[i] (LDS) per OutMode.
// `segs` lives in LDS. Returns false if pre() reported an abort.
//  * ACC64 (bf16 weights only): products and sums in fp64 (bf16 x fp32 products are exact
//    there) and fp64 results, stored to ((double*)out)[i] (OUT_STORE only).
template <bool FP8, int K, int INFL, bool ACC64 = false, typename Pre>
__device__ __forceinline__ bool gemv_list(const RowSeg* segs, int nseg, const float* act, float* out, int mode,
                                          Pre&& pre) {
  static_assert(!(ACC64 && FP8), "fp64 accumulation is for bf16 weights");
  static_assert(!FP8 || K % 64 == 0, "whole 64-element blocks of the padded activation layout");
  using AccT = typename std::conditional<ACC64, double, float>::type;
  using LY = GemvLayout<FP8, K, INFL>;
  constexpr int EPC = LY::EPC, LPR = LY::LPR, CPL = LY::CPL, U = LY::U;
  constexpr int RPW = 64 / LPR;
  constexpr int SBK = (K + 127) / 128;
  constexpr size_t RS = (size_t)K * (FP8 ? 1 : 2);
  const int lane = tid_opaque() & 63, wave = tid_opaque() >> 6;
  const int li = lane % LPR, rsub = lane / LPR;
  int nrows = 0;
  for (int s = 0; s < nseg; s++) nrows += segs[s].n;
  const int groups = (nrows + RPW - 1) / RPW;
  const int iters = (groups + NWAVES - 1) / NWAVES;
  constexpr int STEP = NWAVES * RPW;   // list rows between consecutive rows of one lane
  uint4 buf[U][CPL];
  float sc[FP8 ? U : 1][FP8 ? CPL : 1];
  // Per-lane cursor over the segment list: (segment, row in segment). Rows advance by
  // STEP; crossing into the next segment costs one LDS read of its length. Rows past the
  // end of the list clamp to the last row (their results are discarded).
  struct Cursor {
    int seg, r;
  };
  auto advance = [&](Cursor& c, int by) {
    c.r += by;
    int n = segs[c.seg].n;
    while (c.r >= n && c.seg < nseg - 1) {
      c.r -= n;
      c.seg++;
      n = segs[c.seg].n;
    }
  };
  auto clamp_row = [&](const Cursor& c) { return c.seg == nseg - 1 ? min(c.r, segs[c.seg].n - 1) : c.r; };
  Cursor ci{0, -STEP}, cc{0, -STEP};   // issue cursor runs U rows ahead of the compute cursor
  const int first = wave * RPW + rsub;
  auto issue = [&](int u) {
    const RowSeg& S = segs[ci.seg];
    const int r = clamp_row(ci);
    const uint8_t* p = S.w + (size_t)r * RS + (size_t)li * 16;
#pragma unroll
    for (int j = 0; j < CPL; j++) buf[u][j] = ld_stream16(p + (size_t)j * LPR * 16);
    if constexpr (FP8) {
      const PLD_GLOBAL float* sr = gp(S.s) + (size_t)((S.srow + r) >> 7) * SBK;
#pragma unroll
      for (int j = 0; j < CPL; j++) sc[u][j] = sr[((j * LPR + li) * 16) >> 7];
    }
  };
  if (nrows > 0) {
    ci.r = 0;
    advance(ci, first);
    cc = ci;
#pragma unroll
    for (int u = 0; u < U; u++) {
      issue(u);
      if (u + 1 < U) advance(ci, STEP);
    }
  }
  if (!pre()) return false;
  if (nrows <= 0) return true;
#pragma unroll 1
  for (int it = 0; it < iters; it += U) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int cur = it + u;
      const int i = cur * STEP + first;
      const RowSeg& S = segs[cc.seg];
      const float* a = act + S.act_off;
      const float alpha = S.alpha;
      const int oi = i;
      AccT acc = 0;
#pragma unroll
      for (int j = 0; j < CPL; j++) {
        float at[EPC];
        const float4* ap = reinterpret_cast<const float4*>(a + apad<FP8>((j * LPR + li) * EPC));
#pragma unroll
        for (int q = 0; q < EPC / 4; q++) {
          const float4 t = ap[q];
          at[4 * q] = t.x; at[4 * q + 1] = t.y; at[4 * q + 2] = t.z; at[4 * q + 3] = t.w;
        }
        if constexpr (FP8) acc += sc[u][j] * dot16_fp8(buf[u][j], at);
        else if constexpr (ACC64) acc += dot8_bf16_f64(buf[u][j], at);
        else acc += dot8_bf16(buf[u][j], at);
      }
      if (cur + U < iters) {
        advance(ci, STEP);
        issue(u);
      }
      advance(cc, STEP);
      if constexpr (ACC64) {
        acc = dpp_sum_f64<LPR>(acc);
        if (li == LPR - 1 && cur < iters && oi < nrows) reinterpret_cast<double*>(out)[oi] = acc;
      } else {
        acc = dpp_sum<LPR>(acc);
        if (li == LPR - 1 && cur < iters && oi < nrows) {
          if (mode == OUT_STORE) out[oi] = acc;
          else out[oi] += alpha * acc;
        }
      }
    }
  }
  return true;
}

// Lookup-table (LUT3) weights: a 3-bit index per weight selects one of the eight E4M3
// entries of the codebook of its 8 x 64 block (the Vera Rubin article's "Lookup Table Weight
// Decompression", 3.125 bits per weight); there is no other scale. On gfx950 the lookup is
// done in registers: the three index bit planes of 32 weights (one u32 word per plane) give,
// for j = 0..7, the byte selectors of weights j, j+8, j+16, j+24 by shifts and masks; one
// v_perm_b32 over the block's 8 codebook bytes then yields their 4 E4M3 codes, converted
// to fp32 two at a time by the hardware FP8 converter. Storage of an [out, in] matrix: per
// row and group of 128 weights 48 bytes (plane p = bytes 16p .. 16p+15, word d bit j = bit p
// of the index of weight 32 d + j), codebooks [out/8][in/64][8] bytes.
__device__ __forceinline__ uint32_t lut_sel(uint32_t p0, uint32_t p1, uint32_t p2, int j) {
  return ((p0 >> j) & 0x01010101u) | (((p1 >> j) & 0x01010101u) << 1) | (((p2 >> j) & 0x01010101u) << 2);
}
// dot of the 32 weights of plane word d (codebook dwords cl, ch) with a[0..31], as four
// independent chains (one per byte of the selector) so that the FMAs do not wait on each other
__device__ __forceinline__ float lut_dot32(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t cl, uint32_t ch,
                                           const float* a) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const uint32_t codes = __builtin_amdgcn_perm(ch, cl, lut_sel(p0, p1, p2, j));
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, true);
    s0 = fmaf(lo.x, a[j], s0);
    s1 = fmaf(lo.y, a[j + 8], s1);
    s2 = fmaf(hi.x, a[j + 16], s2);
    s3 = fmaf(hi.y, a[j + 24], s3);
  }
  return (s0 + s1) + (s2 + s3);
}

// gemv_list for LUT3 rows (same contract: segments of rows, results in list order, the
// first loads issued before pre()). A segment's w points at the index bytes of its first
// row (row stride 3K/8), s at the codebook array of its matrix (bytes, reinterpreted), srow
// is the row of w inside that matrix. 16 lanes share a row; a lane owns CPL groups of 128
// weights; the pipeline runs over (row, group) items, D of them in flight (4 loads each).
template <int K, int D, typename Pre>
__device__ __forceinline__ bool gemv_list_lut(const RowSeg* segs, int nseg, const float* act, float* out, int mode,
                                              Pre&& pre) {
  constexpr int GROUPS = K / 128, LPR = 16, CPL = GROUPS / LPR, RPW = 64 / LPR;
  static_assert(K % 128 == 0 && GROUPS % LPR == 0 && D >= 1, "LUT3 row layout");
  constexpr size_t RS = (size_t)K * 3 / 8;    // index bytes per row
  constexpr size_t CBR = (size_t)K / 64 * 8;  // codebook bytes per block of 8 rows
  constexpr int STEP = NWAVES * RPW;
  const int lane = tid_opaque() & 63, wave = tid_opaque() >> 6;
  const int li = lane % LPR, rsub = lane / LPR;
  int nrows = 0;
  for (int s = 0; s < nseg; s++) nrows += segs[s].n;
  const int groups = (nrows + RPW - 1) / RPW;
  const int iters = (groups + NWAVES - 1) / NWAVES;   // rows per lane (past the end: clamped)
  const int nitems = iters * CPL;
  struct Cursor {
    int seg, r;
  };
  auto advance = [&](Cursor& c, int by) {
    c.r += by;
    int n = segs[c.seg].n;
    while (c.r >= n && c.seg < nseg - 1) {
      c.r -= n;
      c.seg++;
      n = segs[c.seg].n;
    }
  };
  auto clamp_row = [&](const Cursor& c) { return c.seg == nseg - 1 ? min(c.r, segs[c.seg].n - 1) : c.r; };
  const int first = wave * RPW + rsub;
  Cursor ci{0, 0}, cc{0, 0};
  int ji = 0;   // group of the issue cursor within its row
  uint4 buf[D][4];
  auto issue = [&](int slot) {
    const RowSeg& S = segs[ci.seg];
    const int r = clamp_row(ci);
    const int g = ji * LPR + li;
    const uint8_t* p = S.w + (size_t)r * RS + (size_t)g * 48;
    buf[slot][0] = ld_stream16(p);
    buf[slot][1] = ld_stream16(p + 16);
    buf[slot][2] = ld_stream16(p + 32);
    buf[slot][3] = ld_stream16(reinterpret_cast<const uint8_t*>(S.s) + (size_t)((S.srow + r) >> 3) * CBR + g * 16);
    if (++ji == CPL) {
      ji = 0;
      advance(ci, STEP);
    }
  };
  if (nrows > 0) {
    advance(ci, first);
    cc = ci;
#pragma unroll
    for (int d = 0; d < D; d++) issue(d);
  }
  if (!pre()) return false;
  if (nrows <= 0) return true;
  float acc = 0.f;
  int jc = 0, row_i = 0;
#pragma unroll 1
  for (int t0 = 0; t0 < nitems; t0 += D) {
#pragma unroll
    for (int d = 0; d < D; d++) {
      const int t = t0 + d;
      if (t < nitems) {   // uniform across the wave
        const int g = jc * LPR + li;
        const float* a = act + segs[cc.seg].act_off + apad<true>(g * 128);
        float part[4];
#pragma unroll
        for (int w = 0; w < 4; w++) {
          float at[32];
#pragma unroll
          for (int q = 0; q < 8; q++) {
            const float4 v = reinterpret_cast<const float4*>(a + apad<true>(32 * w) - apad<true>(0))[q];
            at[4 * q] = v.x; at[4 * q + 1] = v.y; at[4 * q + 2] = v.z; at[4 * q + 3] = v.w;
          }
          const uint32_t p0 = w == 0 ? buf[d][0].x : w == 1 ? buf[d][0].y : w == 2 ? buf[d][0].z : buf[d][0].w;
          const uint32_t p1 = w == 0 ? buf[d][1].x : w == 1 ? buf[d][1].y : w == 2 ? buf[d][1].z : buf[d][1].w;
          const uint32_t p2 = w == 0 ? buf[d][2].x : w == 1 ? buf[d][2].y : w == 2 ? buf[d][2].z : buf[d][2].w;
          const uint32_t cl = w < 2 ? buf[d][3].x : buf[d][3].z, ch = w < 2 ? buf[d][3].y : buf[d][3].w;
          part[w] = lut_dot32(p0, p1, p2, cl, ch, at);
        }
        acc += (part[0] + part[1]) + (part[2] + part[3]);
        if (t + D < nitems) issue(d);
        if (++jc == CPL) {
          jc = 0;
          const float sum = dpp_sum<LPR>(acc);
          const int oi = row_i * STEP + first;
          if (li == LPR - 1 && oi < nrows) {
            if (mode == OUT_STORE) out[oi] = sum;
            else out[oi] += segs[cc.seg].alpha * sum;
          }
          acc = 0.f;
          row_i++;
          advance(cc, STEP);
        }
      }
    }
  }
  return true;
}

struct NoPre {
  __device__ __forceinline__ bool operator()() const { return true; }
};

// Balanced split of n items over g parts: part p gets [split(n,g,p), split(n,g,p+1)).
__host__ __device__ inline int split_at(int n, int g, int p) { return (int)(((long long)n * p) / g); }

}  // namespace pld
