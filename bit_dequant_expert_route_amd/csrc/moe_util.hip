// moe_util.hip -- kernels around the hot path: the stand-alone combine, the
// seeded synthetic-weight fill, the router's column tiles, zeroing and a copy.
#include "moe_internal.h"

#include <stdint.h>

#include <mutex>

namespace moe_impl {

thread_local LaunchEvents g_launch_events;

// ---------------------------------------------------------------------------
// the workspace of the no-allocation entry point: one array per GPU the
// library runs on, held until the process ends.  Host code never passes the
// array's name to a kernel (in host code it is only a stand-in): each device's
// address is looked up once, with that device current, and kept here.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}


// ---------------------------------------------------------------------------
// elementwise combine (stand-alone entry point)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_combine(CombineParams p) {
  const int o = blockIdx.x * kBlock + threadIdx.x;
  if (o >= p.H) return;
  float acc = p.h_res[o];
  for (int k = 0; k < p.K; ++k) acc = fmaf(p.w[k], p.y[(size_t)k * p.H + o], acc);
  acc = fmaf(p.sigma[0], p.y_shared[o], acc);
  p.out[o] = acc;
}

// ---------------------------------------------------------------------------
// synthetic weights: SplitMix64 used counter-style (Steele, Lea and Flood,
// OOPSLA 2014), see moe_fill_experts in include/moe.h
// ---------------------------------------------------------------------------
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kRoot = 0x6D6F652D67656E31ull;

__device__ __forceinline__ uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__device__ __forceinline__ uint64_t sm_out(uint64_t key, uint64_t i) {
  return sm_mix(key + (i + 1) * kGamma);
}

// fp64 -> bf16 bits, round to nearest even from the full significand
__device__ __forceinline__ uint32_t f64_to_bf16(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t sign = (uint32_t)(b >> 63);
  if ((b << 1) == 0) return sign << 15;
  const int e = (int)((b >> 52) & 0x7FF);
  const uint64_t m = (b & ((1ull << 52) - 1)) | (1ull << 52);
  uint64_t keep = m >> 45;
  const uint64_t rem = m & ((1ull << 45) - 1);
  const uint64_t half = 1ull << 44;
  if (rem > half || (rem == half && (keep & 1))) ++keep;
  int exp = e - 1023 + 127;
  if (keep == 256) {
    keep = 128;
    ++exp;
  }
  return (sign << 15) | ((uint32_t)exp << 7) | (uint32_t)(keep & 0x7F);
}

__device__ __forceinline__ uint32_t uniform_bf16(uint32_t u24, double lo, double hi) {
  const double t = ((double)u24 + 0.5) * (1.0 / 16777216.0);
  const double d = __dsub_rn(hi, lo);
  const double v = __dadd_rn(lo, __dmul_rn(d, t));
  return f64_to_bf16(v);
}

__global__ __launch_bounds__(kBlock) void k_fill(FillParams p) {
  const int j = blockIdx.y;
  uint8_t *rec = p.dst + (size_t)j * p.stride;
  const uint64_t ng = (uint64_t)p.I * p.H * p.bits / 32;  // words of gate (= up)
  const uint64_t nd = ng;                                  // words of down
  const uint64_t gg = (uint64_t)p.I * (p.H / 64);          // sb words of gate (= up)
  const uint64_t gd = (uint64_t)p.H * (p.I / 64);          // sb words of down
  const uint64_t n_units[6] = {ng / 2, ng / 2, nd / 2, gg, gg, gd};
  const size_t offs[6] = {p.off.gate_codes, p.off.up_codes, p.off.down_codes,
                          p.off.gate_sb, p.off.up_sb, p.off.down_sb};
  uint64_t base = sm_out(sm_out(sm_out(kRoot, p.seed), (uint64_t)p.layer),
                         (uint64_t)(p.first_expert + j));
  uint64_t total = 0;
  for (int s = 0; s < 6; ++s) total += n_units[s];
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += stride) {
    int s = 0;
    uint64_t i = u;
    while (i >= n_units[s]) {
      i -= n_units[s];
      ++s;
    }
    const uint64_t key = sm_out(base, (uint64_t)s);
    const uint64_t r = sm_out(key, i);
    if (s < 3) {
      uint2 *dst = reinterpret_cast<uint2 *>(rec + offs[s]) + i;
      *dst = make_uint2((uint32_t)r, (uint32_t)(r >> 32));
    } else {
      const uint32_t us = (uint32_t)(r >> 40);
      const uint32_t ub = (uint32_t)((r >> 16) & 0xFFFFFFu);
      const uint32_t sbits = uniform_bf16(us, p.scale_lo, p.scale_hi);
      const uint32_t bbits = uniform_bf16(ub, p.bias_lo, p.bias_hi);
      reinterpret_cast<uint32_t *>(rec + offs[s])[i] = sbits | (bbits << 16);
    }
  }
}

__global__ __launch_bounds__(kBlock) void k_zero(uint8_t *ptr, size_t bytes) {
  const size_t n16 = bytes / 16;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    reinterpret_cast<uint4 *>(ptr)[i] = make_uint4(0, 0, 0, 0);
  const size_t tail = bytes - n16 * 16;
  if (blockIdx.x == 0 && threadIdx.x < tail) ptr[n16 * 16 + threadIdx.x] = 0;
}

__global__ __launch_bounds__(kBlock) void k_copy_f32(float *dst, const float *src, int n) {
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

// router column tiles: thread i copies the 8 columns of expert e = i mod E in
// tile t = i / E (8 * esz bytes, as 16-byte words)
__global__ __launch_bounds__(kBlock) void k_router_tile(const uint8_t *router, int E, int H, int esz,
                                                        uint8_t *out) {
  const size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
  const size_t n = (size_t)E * (H / 8);
  if (i >= n) return;
  const int e = (int)(i % E);
  const size_t t = i / E;
  const uint4 *src = reinterpret_cast<const uint4 *>(router + ((size_t)e * H + t * 8) * esz);
  uint4 *dst = reinterpret_cast<uint4 *>(out + i * 8 * esz);
  for (int w = 0; w < esz / 2; ++w) dst[w] = src[w];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_router_tile(const void *router, int E, int H, int esz, void *out, hipStream_t s) {
  const size_t n = (size_t)E * (H / 8);
  if (n == 0) return hipSuccess;
  MOE_LAUNCH(k_router_tile, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, s,
             static_cast<const uint8_t *>(router), E, H, esz, static_cast<uint8_t *>(out));
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams &p, hipStream_t s) {
  MOE_LAUNCH(k_combine, dim3((p.H + kBlock - 1) / kBlock), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fill(const FillParams &p, hipStream_t s) {
  const dim3 grid(1024, p.n);
  MOE_LAUNCH(k_fill, grid, dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_zero(void *ptr, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  size_t blocks = (bytes / 16 + kBlock - 1) / kBlock;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  MOE_LAUNCH(k_zero, dim3((unsigned)blocks), dim3(kBlock), 0, s,
                     static_cast<uint8_t *>(ptr), bytes);
  return hipGetLastError();
}

hipError_t launch_copy_f32(float *dst, const float *src, int n, hipStream_t s) {
  MOE_LAUNCH(k_copy_f32, dim3((n + kBlock - 1) / kBlock), dim3(kBlock), 0, s, dst, src, n);
  return hipGetLastError();
}

}  // namespace moe_impl
