// Measurement program (not part of libmsa.so): the fp8 matrix-core rate that
// three instruction mixes sustain on gfx950, on constant and on random E4M3
// operands.  It sets the practical ceiling the scorer's roofline fraction is
// read against: MI355X's 5.0 PFLOP/s dense fp8 peak assumes the full engine
// clock, which the chip holds only while few operand bits toggle.
//
//   chain_regs    products chained into 4 accumulators, operands in registers
//   chain_lds     the same, the 16-token fragments read from a 16 KiB page in
//                 LDS (the scorer's swizzled layout, 16 waves, 4 query tiles
//                 per wave sharing each fragment)
//   page_max_lds  the scorer's page loop without its epilogue: zero-initialised
//                 products, running max3 per query tile, the page max summed
//
// Every kernel reads and writes only its own buffers (grid and indexing are
// fixed below).  Prints one line per variant: TFLOP/s and the fraction of
// 5.0 PFLOP/s, from HIP events around 5 launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ v8i frag(const uint8_t* p0, const uint8_t* p1) {
  const uint4 x = *reinterpret_cast<const uint4*>(p0);
  const uint4 y = *reinterpret_cast<const uint4*>(p1);
  return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}

constexpr int kSrcBytes = 131072;       // 64 KiB of pages + 64 KiB of query rows
constexpr double kFlopPerMfma = 16.0 * 16 * 128 * 2;

// 256 threads; per iteration 16 products (4 fragments x 4 query tiles).
__global__ __launch_bounds__(256) void chain_regs(const uint8_t* __restrict__ src,
                                                  float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  v8i a[4], b[4];
  for (int j = 0; j < 4; ++j) {
    a[j] = frag(src + (lane * 256 + j * 32) % 65536, src + (lane * 256 + j * 32 + 16) % 65536);
    b[j] = frag(src + 65536 + lane * 128 + j * 32 % 128, src + 65536 + lane * 128 + 16);
  }
  v4f c[4] = {};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int n = 0; n < 4; ++n) c[n] = mfma(a[j], b[n], c[n]);
  float s = 0.f;
  for (int n = 0; n < 4; ++n) s += c[n][0] + c[n][1] + c[n][2] + c[n][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// 1024 threads (16 waves), 64 KiB of LDS (4 pages); per page and wave 32
// products (8 token tiles x 4 query tiles).  MODE 0: chained, 1: page max.
template <int MODE>
__global__ __launch_bounds__(1024) void page_loop(const uint8_t* __restrict__ src,
                                                  float* __restrict__ out, int pages) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[65536];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  for (int i = tid; i < 65536 / 16; i += 1024)
    reinterpret_cast<uint4*>(lds)[i] = reinterpret_cast<const uint4*>(src)[i];
  v8i qf[4];
  for (int n = 0; n < 4; ++n) {
    const uint8_t* q = src + 65536 + ((wave * 64 + n * 16 + col) * 128) % 65536 + grp * 32;
    qf[n] = frag(q, q + 16);
  }
  __syncthreads();
  // rows of 8 pieces of 16 bytes, piece c of row t at c ^ ((t >> 1) & 7)
  const int sw = (col >> 1) & 7;
  const int off0 = 16 * ((2 * grp) ^ sw), off1 = 16 * ((2 * grp + 1) ^ sw);
  v4f acc[4] = {};
  float s = 0.f;
  for (int p = 0; p < pages; ++p) {
    const uint8_t* pg = lds + (p & 3) * 16384;
    if constexpr (MODE == 0) {
#pragma unroll
      for (int T = 0; T < 8; ++T) {
        const uint8_t* row = pg + (T * 16 + col) * 128;
        const v8i a = frag(row + off0, row + off1);
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[n] = mfma(a, qf[n], acc[n]);
      }
    } else {
      v4f rmax[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) rmax[n] = v4f{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int T = 0; T < 8; ++T) {
        const uint8_t* row = pg + (T * 16 + col) * 128;
        const v8i a = frag(row + off0, row + off1);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const v4f x = mfma(a, qf[n], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int i = 0; i < 4; ++i) rmax[n][i] = fmaxf(rmax[n][i], x[i]);
        }
      }
#pragma unroll
      for (int n = 0; n < 4; ++n) s += fmaxf(fmaxf(rmax[n][0], rmax[n][1]), fmaxf(rmax[n][2], rmax[n][3]));
    }
  }
  for (int n = 0; n < 4; ++n) s += acc[n][0] + acc[n][1] + acc[n][2] + acc[n][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

#define CHECK(x)                                                                     \
  do {                                                                               \
    hipError_t e_ = (x);                                                             \
    if (e_ != hipSuccess) {                                                          \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));            \
      std::exit(1);                                                                  \
    }                                                                                \
  } while (0)

template <class Launch>
void timed(const char* name, const char* data, double flop_per_launch, Launch&& launch) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  launch();
  CHECK(hipEventRecord(e0));
  const int reps = 5;
  for (int r = 0; r < reps; ++r) launch();
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  const double tf = flop_per_launch * reps / (ms * 1e-3) / 1e12;
  std::printf("%-13s %-8s %.3f ms/launch  %7.1f TFLOP/s  %.3f of 5000\n", name, data, ms / reps, tf,
              tf / 5000.0);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
}

}  // namespace

int main() {
  uint8_t* src = nullptr;
  float* out = nullptr;
  CHECK(hipMalloc(&src, kSrcBytes));
  CHECK(hipMalloc(&out, 1024 * 1024 * sizeof(float)));
  // random E4M3 codes with magnitudes in [2^-3, 2^5] (no NaN codes), from a
  // fixed linear congruential sequence
  std::vector<uint8_t> rnd(kSrcBytes);
  uint32_t x = 12345u;
  for (auto& c : rnd) {
    x = x * 1664525u + 1013904223u;
    uint8_t v = (uint8_t)(x >> 24);
    if ((v & 0x78) < 0x20) v |= 0x30;
    if ((v & 0x78) > 0x60) v &= 0xDF;
    c = v;
  }
  const std::vector<uint8_t> one(kSrcBytes, 0x38);   // E4M3 1.0
  const int blocks_r = 1024, iters = 5000, pages = 2000;
  const double f_regs = (double)blocks_r * 4 * iters * 16 * kFlopPerMfma;
  const double f_page = 256.0 * 16 * pages * 32 * kFlopPerMfma;
  // clock ramp
  CHECK(hipMemcpy(src, one.data(), kSrcBytes, hipMemcpyHostToDevice));
  for (int i = 0; i < 10; ++i) hipLaunchKernelGGL(chain_regs, dim3(blocks_r), dim3(256), 0, 0, src, out, iters);
  CHECK(hipDeviceSynchronize());
  for (int d = 0; d < 2; ++d) {
    const char* data = d == 0 ? "constant" : "random";
    CHECK(hipMemcpy(src, d == 0 ? one.data() : rnd.data(), kSrcBytes, hipMemcpyHostToDevice));
    timed("chain_regs", data, f_regs, [&] {
      hipLaunchKernelGGL(chain_regs, dim3(blocks_r), dim3(256), 0, 0, src, out, iters);
    });
    timed("chain_lds", data, f_page, [&] {
      hipLaunchKernelGGL(page_loop<0>, dim3(256), dim3(1024), 0, 0, src, out, pages);
    });
    timed("page_max_lds", data, f_page, [&] {
      hipLaunchKernelGGL(page_loop<1>, dim3(256), dim3(1024), 0, 0, src, out, pages);
    });
  }
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  CHECK(hipFree(src));
  CHECK(hipFree(out));
  return 0;
}
