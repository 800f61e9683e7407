// Device building blocks of the persistent decode kernel (gfx950, wave64).
//
// Synchronisation protocol (measured on MI355X before it was chosen):
//  * Cross-workgroup data (activations, attention partials, appended cache rows) is
//    written with agent-scope relaxed atomic stores, which write through to the
//    device coherence point, and read back with agent-scope relaxed atomic loads.
//    No L2 write-back or invalidate is needed per stage; weights use ordinary
//    (non-temporal) loads because they are never written.
//  * A producer workgroup waits for its own stores (s_waitcnt vmcnt(0) in every
//    wave), passes a workgroup barrier, and one thread bumps a per-XCD counter; the
//    last arriver of each XCD group bumps the stage's global counter. Consumers poll
//    the global counter. A grid-wide dependency costs about 2.8 us this way, versus
//    ~10 us for one flat counter with release/acquire fences.
//  * Only static weights may be loaded before a wait; activations are always read
//    after it. This is the ordering rule the vLLM Kimi K3 backend article reports
//    from its kernel audit (section "Agent-written kernels face evidence gates").
//  * Every wait is bounded by a wall-clock deadline; on expiry the workgroup records
//    a status word, raises a global abort flag and leaves, and so do all others.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pld {

constexpr int BLOCK = 512;
constexpr int NWAVES = BLOCK / 64;
constexpr int NXCD = 8;
constexpr int CTR_STRIDE = 64;       // uint32 words between counters (256 B)

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
__device__ __forceinline__ void st_f64(double* p, double v) {
  __hip_atomic_store(gp(reinterpret_cast<uint64_t*>(p)), (uint64_t)__double_as_longlong(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double ld_f64(const double* p) {
  return __longlong_as_double((long long)__hip_atomic_load(gp(reinterpret_cast<uint64_t*>(const_cast<double*>(p))),
                                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ uint32_t atomic_add_u32(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// ----------------------------------------------------------------- reductions
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
  return v;
}
// Block-wide sum in a fixed order (wave sums, then wave 0..7 in order). All threads get the result.
template <typename T>
__device__ __forceinline__ T block_sum(T v, T* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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

// Lane layout per reduction length K (elements) and weight format, fixed at compile time:
// LPR lanes per row, CPL 16-byte chunks per lane and row, U rows in flight per wave.
template <bool FP8, int K>
struct GemvLayout {
  static constexpr int EPC = FP8 ? 16 : 8;
  static constexpr int CHUNKS = K / EPC;
  static constexpr int LPR = CHUNKS >= 64 ? 64 : CHUNKS;
  static constexpr int CPL = CHUNKS / LPR;
  static constexpr int U = CPL >= 4 ? 2 : (CPL >= 2 ? 4 : 8);
  static_assert(K % EPC == 0 && CHUNKS % LPR == 0 && (LPR == 16 || LPR == 32 || LPR == 64), "unsupported K");
};

// Streams rows [r0, r1) of a [rows, K] weight matrix against an fp32 activation vector
// in LDS.
//  * LPR lanes share one row (64/LPR rows per wave pass); each lane reads CPL 16-byte
//    chunks per row, chunk j of lane l covering elements [(j*LPR + l) * EPC, +EPC);
//  * a wave keeps U rows of loads in flight (U*CPL 16-byte loads per lane);
//  * the first U rows are issued BEFORE `pre()` runs -- pre is where the caller waits
//    for its dependency and stages the activation into LDS -- so the wait overlaps with
//    the first weight bytes arriving; only static weights are loaded ahead of a wait;
//  * partial sums are reduced across the LPR lanes and the row's first lane writes the
//    result into `out` (LDS) per OutMode.
// Returns false if pre() reported an abort.
template <bool FP8, int K, typename ACC, typename Pre>
__device__ __forceinline__ bool gemv(const uint8_t* __restrict__ W, const float* __restrict__ S, int r0, int r1,
                                     const float* act, ACC* out, int mode, float alpha, Pre&& pre) {
  using LY = GemvLayout<FP8, K>;
  constexpr int EPC = LY::EPC, LPR = LY::LPR, CPL = LY::CPL, U = LY::U;
  constexpr int RPW = 64 / LPR;
  constexpr int SBK = (K + 127) / 128;
  // activations stay in registers when they fit beside the in-flight loads, else they
  // are re-read from LDS per chunk (ds_read_b128, 2-4 LDS bytes per weight byte)
  constexpr bool AREG = CPL * EPC <= 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane % LPR, rsub = lane / LPR;
  const int nrows = r1 - r0;
  const int groups = (nrows + RPW - 1) / RPW;
  const int iters = (groups + NWAVES - 1) / NWAVES;
  constexpr size_t RS = (size_t)K * (FP8 ? 1 : 2);
  uint4 buf[U][CPL];
  float sc[FP8 ? U : 1][FP8 ? CPL : 1];
  // rows past r1 re-read the last valid row (results discarded): no predicated loads
  auto issue = [&](int it, int u) {
    const int r = min(r0 + (it * NWAVES + wave) * RPW + rsub, r1 - 1);
    const uint8_t* p = W + (size_t)r * RS + (size_t)li * 16;
#pragma unroll
    for (int j = 0; j < CPL; j++) buf[u][j] = ld_stream16(p + (size_t)j * LPR * 16);
    if constexpr (FP8) {
      const PLD_GLOBAL float* sr = gp(S) + (size_t)(r >> 7) * SBK;
#pragma unroll
      for (int j = 0; j < CPL; j++) sc[u][j] = sr[((j * LPR + li) * 16) >> 7];
    }
  };
  if (nrows > 0) {
#pragma unroll
    for (int u = 0; u < U; u++) issue(u, u);
  }
  if (!pre()) return false;
  if (nrows <= 0) return true;
  float av[AREG ? CPL : 1][AREG ? EPC : 1];
  if constexpr (AREG) {
#pragma unroll
    for (int j = 0; j < CPL; j++) {
      const float4* ap = reinterpret_cast<const float4*>(act + (j * LPR + li) * EPC);
#pragma unroll
      for (int q = 0; q < EPC / 4; q++) {
        const float4 t = ap[q];
        av[j][4 * q] = t.x; av[j][4 * q + 1] = t.y; av[j][4 * q + 2] = t.z; av[j][4 * q + 3] = t.w;
      }
    }
  }
#pragma unroll 1
  for (int it = 0; it < iters; it += U) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int cur = it + u;
      ACC acc = 0;
#pragma unroll
      for (int j = 0; j < CPL; j++) {
        float atmp[EPC];
        const float* aj;
        if constexpr (AREG) {
          aj = av[j];
        } else {
          const float4* ap = reinterpret_cast<const float4*>(act + (j * LPR + li) * EPC);
#pragma unroll
          for (int q = 0; q < EPC / 4; q++) {
            const float4 t = ap[q];
            atmp[4 * q] = t.x; atmp[4 * q + 1] = t.y; atmp[4 * q + 2] = t.z; atmp[4 * q + 3] = t.w;
          }
          aj = atmp;
        }
        if constexpr (FP8) {
          acc += (ACC)(sc[u][j] * dot16_fp8(buf[u][j], aj));
        } else if constexpr (sizeof(ACC) == 8) {
          acc += dot8_bf16_f64(buf[u][j], aj);
        } else {
          acc += dot8_bf16(buf[u][j], aj);
        }
      }
      if (cur + U < iters) issue(cur + U, u);
#pragma unroll
      for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
      const int r = r0 + (cur * NWAVES + wave) * RPW + rsub;
      if (li == 0 && cur < iters && r < r1) {
        if (mode == OUT_STORE) out[r - r0] = acc;
        else out[r - r0] += (ACC)alpha * acc;
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
