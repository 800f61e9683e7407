// Device half of the seeded input generator (the host half is synth/gen.py; the two
// follow one written definition and a GPU test checks they write identical bytes).
// It fills weights, caches and input vectors directly in device memory so that the
// large workloads (tens to hundreds of GB of weights) never cross PCIe. It contains
// none of the decode method's arithmetic.
//
// Definition (see synth/gen.py for the full text):
//   key   = mix(seed*G + mix(tid*G + G)),  r_i = mix(key + (i+1)*G)   (SplitMix64 mixer)
//   n_i   = fp32(l0+l1+l2+l3 - 131070) * INV_SIGMA   (four 16-bit lanes of r_i)
//   v     = n*std  or  (n*std)+mean                   (separate correctly rounded fp32 ops)
//   bf16  = round-to-nearest-even of v
//   FP8   = E4M3FN of clamp(v/scale, +-448), scale = amax/448 per 128x128 block (or per row)
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t G = 0x9E3779B97F4A7C15ull;
constexpr float INV_SIGMA = 0x1.bb67aep-16f;

__device__ __host__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__device__ __host__ inline uint64_t stream_key(uint64_t seed, uint64_t tid) { return mix64(seed * G + mix64(tid * G + G)); }

__device__ inline float normal_at(uint64_t key, uint64_t i) {
  const uint64_t r = mix64(key + (i + 1) * G);
  const int64_t s = (int64_t)((r & 0xFFFF) + ((r >> 16) & 0xFFFF) + ((r >> 32) & 0xFFFF) + (r >> 48)) - 131070;
  return __fmul_rn((float)s, INV_SIGMA);
}
__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
// E4M3FN code of a value already clamped to [-448, 448] (hardware conversion, RNE)
__device__ inline uint8_t e4m3(float q) {
  const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(q, 0.0f, 0, false);
  return (uint8_t)(packed & 0xff);
}

// out[(h*d1s + p)*d2 + c] = bf16(normal(((h<<20)|p)*d2 + c) * std) for h<d0, p<d1, c<d2
__global__ void k_bf16_3d(uint16_t* out, int d0, int d1, int d1s, int d2, uint64_t key, float stdv) {
  const int64_t total = (int64_t)d0 * d1 * d2;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(e % d2);
    const int64_t hp = e / d2;
    const int p = (int)(hp % d1), h = (int)(hp / d1);
    const uint64_t gi = ((((uint64_t)h) << 20) | (uint64_t)p) * (uint64_t)d2 + (uint64_t)c;
    out[((int64_t)h * d1s + p) * d2 + c] = bf16_rne(__fmul_rn(normal_at(key, gi), stdv));
  }
}

__global__ void k_f32(float* out, int64_t n, uint64_t key, float stdv, float mean, int has_mean) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    float v = __fmul_rn(normal_at(key, (uint64_t)e), stdv);
    if (has_mean) v = __fadd_rn(v, mean);
    out[e] = v;
  }
}

// One workgroup (256 threads) per 128x128 block of a [rows, cols] matrix.
__global__ void __launch_bounds__(256) k_fp8_block(uint8_t* codes, float* scales, int rows, int cols, uint64_t key,
                                                    float stdv, int row_offset) {
  const int nbi = (cols + 127) / 128;
  const int bo = blockIdx.x / nbi, bi = blockIdx.x % nbi;
  const int r0 = bo * 128, c0 = bi * 128;
  const int rn = min(128, rows - r0), cn = min(128, cols - c0);
  __shared__ float red[256];
  float amax = 0.f;
  for (int e = threadIdx.x; e < rn * cn; e += 256) {
    const int r = r0 + e / cn, c = c0 + e % cn;
    const float v = __fmul_rn(normal_at(key, (uint64_t)(r + row_offset) * (uint64_t)cols + c), stdv);
    amax = fmaxf(amax, fabsf(v));
  }
  red[threadIdx.x] = amax;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  amax = red[0];
  const float sc = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  if (threadIdx.x == 0) scales[blockIdx.x] = sc;
  for (int e = threadIdx.x; e < rn * cn; e += 256) {
    const int r = r0 + e / cn, c = c0 + e % cn;
    const float v = __fmul_rn(normal_at(key, (uint64_t)(r + row_offset) * (uint64_t)cols + c), stdv);
    const float q = fminf(fmaxf(__fdiv_rn(v, sc), -448.0f), 448.0f);
    codes[(int64_t)r * cols + c] = e4m3(q);
  }
}

// Cache rows of FP8 keys with one scale per row: element index (p*d + c), one wave per row.
__global__ void __launch_bounds__(64) k_fp8_rows(uint8_t* codes, float* scales, int n_rows, int d, uint64_t key,
                                                  float stdv) {
  const int p = blockIdx.x;
  if (p >= n_rows) return;
  float amax = 0.f;
  for (int c = threadIdx.x; c < d; c += 64)
    amax = fmaxf(amax, fabsf(__fmul_rn(normal_at(key, (uint64_t)p * d + c), stdv)));
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float sc = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  if (threadIdx.x == 0) scales[p] = sc;
  for (int c = threadIdx.x; c < d; c += 64) {
    const float v = __fmul_rn(normal_at(key, (uint64_t)p * d + c), stdv);
    codes[(int64_t)p * d + c] = e4m3(fminf(fmaxf(__fdiv_rn(v, sc), -448.0f), 448.0f));
  }
}

// LUT3 matrices [rows, cols] (rows % 8 == 0, cols % 128 == 0): one thread per (row, group of
// 128 weights) writes the group's three 16-byte index planes; one thread per 8x64 block
// writes its 8 codebook codes. Same definition as synth/gen.py (lut3_matrix).
__constant__ float LUT_Z[8] = {-1.5341205f, -0.88714653f, -0.48877642f, -0.15731068f,
                               0.15731068f, 0.48877642f, 0.88714653f, 1.5341205f};
__global__ void k_lut3(uint8_t* idx, uint8_t* cb, int rows, int cols, uint64_t key, float stdv) {
  const int64_t n_groups = (int64_t)rows * (cols / 128);
  const int64_t n_blocks = (int64_t)(rows / 8) * (cols / 64);
  const int64_t n_w = (int64_t)rows * cols;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n_groups + n_blocks;
       e += (int64_t)gridDim.x * blockDim.x) {
    if (e < n_groups) {
      const int64_t row = e / (cols / 128), g = e % (cols / 128);
      uint32_t w[3][4] = {};
      for (int d = 0; d < 4; d++)
        for (int j = 0; j < 32; j++) {
          const uint64_t i = (uint64_t)(row * cols + g * 128 + 32 * d + j);
          const uint32_t v = (uint32_t)(mix64(key + (i + 1) * G) & 7u);
          for (int p = 0; p < 3; p++) w[p][d] |= ((v >> p) & 1u) << j;
        }
      uint32_t* dst = reinterpret_cast<uint32_t*>(idx + row * (int64_t)(3 * cols / 8) + g * 48);
      for (int p = 0; p < 3; p++)
        for (int d = 0; d < 4; d++) dst[4 * p + d] = w[p][d];
    } else {
      const int64_t b = e - n_groups;
      const uint64_t r = mix64(key + ((uint64_t)(n_w + b) + 1) * G);
      const float u = __fmul_rn((float)(r >> 40), 0x1p-24f);
      const float spread = __fadd_rn(0.75f, __fmul_rn(u, 0.5f));
      for (int k = 0; k < 8; k++) cb[b * 8 + k] = e4m3(__fmul_rn(__fmul_rn(stdv, LUT_Z[k]), spread));
    }
  }
}

int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

extern "C" {

// All functions enqueue on `stream` and return a hipError_t value (0 = success).
int synth_fill_bf16_3d(void* out, int d0, int d1, int d1_stride, int d2, uint64_t seed, uint64_t tid, float stdv,
                       void* stream) {
  if (!out || d0 < 0 || d1 < 0 || d2 <= 0 || d1_stride < d1 || d1 >= (1 << 20)) return (int)hipErrorInvalidValue;
  const int64_t n = (int64_t)d0 * d1 * d2;
  if (n == 0) return 0;
  k_bf16_3d<<<grid_for(n), 256, 0, (hipStream_t)stream>>>((uint16_t*)out, d0, d1, d1_stride, d2, stream_key(seed, tid),
                                                           stdv);
  return (int)hipGetLastError();
}

int synth_fill_f32(void* out, int64_t n, uint64_t seed, uint64_t tid, float stdv, float mean, int has_mean,
                   void* stream) {
  if (!out || n < 0) return (int)hipErrorInvalidValue;
  if (n == 0) return 0;
  k_f32<<<grid_for(n), 256, 0, (hipStream_t)stream>>>((float*)out, n, stream_key(seed, tid), stdv, mean, has_mean);
  return (int)hipGetLastError();
}

// codes [rows, cols] bytes, scales [ceil(rows/128)][ceil(cols/128)] fp32
int synth_fill_fp8_block(void* codes, void* scales, int rows, int cols, uint64_t seed, uint64_t tid, float stdv,
                         void* stream) {
  if (!codes || !scales || rows <= 0 || cols <= 0) return (int)hipErrorInvalidValue;
  const int nb = ((rows + 127) / 128) * ((cols + 127) / 128);
  k_fp8_block<<<nb, 256, 0, (hipStream_t)stream>>>((uint8_t*)codes, (float*)scales, rows, cols, stream_key(seed, tid),
                                                   stdv, 0);
  return (int)hipGetLastError();
}

int synth_fill_lut3(void* idx, void* cb, int rows, int cols, uint64_t seed, uint64_t tid, float stdv, void* stream) {
  if (rows % 8 || cols % 128) return (int)hipErrorInvalidValue;
  const int64_t n = (int64_t)rows * (cols / 128) + (int64_t)(rows / 8) * (cols / 64);
  k_lut3<<<grid_for(n), 256, 0, (hipStream_t)stream>>>((uint8_t*)idx, (uint8_t*)cb, rows, cols, stream_key(seed, tid),
                                                       stdv);
  return (int)hipGetLastError();
}

int synth_fill_fp8_rows(void* codes, void* scales, int n_rows, int d, uint64_t seed, uint64_t tid, float stdv,
                        void* stream) {
  if (!codes || !scales || n_rows < 0 || d <= 0) return (int)hipErrorInvalidValue;
  if (n_rows == 0) return 0;
  k_fp8_rows<<<n_rows, 64, 0, (hipStream_t)stream>>>((uint8_t*)codes, (float*)scales, n_rows, d, stream_key(seed, tid),
                                                     stdv);
  return (int)hipGetLastError();
}

}  // extern "C"
