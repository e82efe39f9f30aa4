// Attainable rates of the instruction mixes the kernels are built from, on
// the GPU it runs on (a standalone program, not part of the library):
//
//   * LDS fragment reads: 16-byte reads of XOR-swizzled 128-byte rows, eight
//     waves per CU (the prefill GEMMs' fragment reads);
//   * FP8 MFMA (16x16x128, f8f6f4) with the products accumulated in place,
//     sixteen independent accumulators per wave, eight waves per CU;
//   * the 128x128 block-scaled FP8 pattern: each MFMA result formed from
//     zero and added to its accumulator with one FMA per element (the
//     product of a per-row activation scale and a weight-block scale),
//     groups of four MFMAs with each group's scaling issued after the next
//     group's MFMAs, as in the prefill GEMM's main loop;
//   * HBM reads: a contiguous non-temporal stream, and the decode GEMMs'
//     fragment pattern (16 weight rows x 64 bytes per load instruction,
//     the K range split over four waves), each after a read of a 1 GiB
//     buffer so the caches hold clean lines.
//
// Every access stays inside its buffer; each kernel's result is consumed
// so the work is not removed.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));     \
      return 1;                                                               \
    }                                                                         \
  } while (0)

__device__ inline int swz(int row, int chunk) { return row * 128 + 16 * (chunk ^ (row & 7)); }

__device__ inline f32x4 mfma8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

constexpr int WG = 512;           // eight waves
constexpr int LDS_BYTES = 49152;  // three 16 KB stages of 128 rows x 128 B

__global__ void __launch_bounds__(WG) k_lds(int iters, int* out) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < LDS_BYTES / 4; i += WG) ((int*)lds)[i] = i;
  __syncthreads();
  const int r16 = lane & 15, lg = lane >> 4;
  i32x4 x = {0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
    const uint8_t* st = lds + (it % 3) * 16384;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int row = ((wave & 1) * 64 + t * 16 + r16) & 127;
      x ^= *(const i32x4*)(st + swz(row, lg));
      x ^= *(const i32x4*)(st + swz(row, lg + 4));
    }
  }
  out[blockIdx.x * WG + tid] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

// SCALED = false: acc[c][t] += A[c] B[t] in the MFMA; true: the block-scaled
// pattern (zero-initialised MFMA, then acc += d * s per element)
template <bool SCALED>
__global__ void __launch_bounds__(WG) k_mfma(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  i32x8 a[4], b[4];
  for (int c = 0; c < 4; ++c) {
    a[c] = (i32x8){lane + c, 0x01010101, 0x02020202, 0x03030303, 4, 5, 6, 7};
    b[c] = (i32x8){7, 6, 5, 4, 0x03030303, 0x02020202, c, lane};
  }
  f32x4 acc[4][4], d[2][4];
  for (int c = 0; c < 4; ++c)
    for (int t = 0; t < 4; ++t) acc[c][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const float s[4] = {1.0f + lane, 2.0f + lane, 3.0f * lane, 4.0f - lane};
  for (int it = 0; it < iters; ++it) {
    if constexpr (!SCALED) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[c][t] = mfma8(a[c], b[t], acc[c][t]);
    } else {
#pragma unroll
      for (int c = 0; c <= 4; ++c) {
        if (c < 4) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int t = 0; t < 4; ++t) d[c & 1][t] = mfma8(a[c], b[t], (f32x4){0.f, 0.f, 0.f, 0.f});
          __builtin_amdgcn_sched_barrier(0);
        }
        if (c > 0) {
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[c - 1][t] += d[(c - 1) & 1][t] * s[t];
        }
      }
    }
    a[0][0] += 1;
    a[2][3] += 1;
  }
  f32x4 r = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < 4; ++c)
    for (int t = 0; t < 4; ++t) r += acc[c][t];
  *(f32x4*)(out + (blockIdx.x * WG + threadIdx.x) * 4) = r;
}

__global__ void __launch_bounds__(256) k_read_all(const i32x4* src, size_t n16, int* out) {
  i32x4 acc = {0, 0, 0, 0};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) acc ^= src[i];
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x5a5a5a5a) out[0] = 1;
}

__global__ void __launch_bounds__(256) k_stream(const i32x4* src, size_t n16, int* out) {
  constexpr int U = 4;
  i32x4 acc = {0, 0, 0, 0};
  const size_t stride = (size_t)gridDim.x * 256 * U;
  for (size_t i = (size_t)blockIdx.x * 256 * U + threadIdx.x; i < n16; i += stride) {
    i32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = i + u * 256 < n16 ? __builtin_nontemporal_load(src + i + u * 256) : (i32x4){0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x5a5a5a5a) out[0] = 1;
}

// one workgroup per 16 weight rows of K bytes; wave w reads K bytes
// [wK/4, (w+1)K/4) of them, two K steps of 128 bytes per batch; a lane
// reads row l%16, bytes 16(l/16) and 64 + 16(l/16) of each step
__global__ void __launch_bounds__(256) k_fragments(const uint8_t* w, int K, int* out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, lg = lane >> 4;
  const uint8_t* row = w + ((size_t)blockIdx.x * 16 + r16) * K;
  const int kw = K / 4, kb = wave * kw;
  i32x4 acc = {0, 0, 0, 0};
  for (int k0 = kb; k0 < kb + kw; k0 += 256) {
    i32x4 v[4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ks = k0 + 128 * u;
      const bool in = ks < kb + kw;
      v[2 * u] = in ? *(const i32x4*)(row + ks + 16 * lg) : (i32x4){0, 0, 0, 0};
      v[2 * u + 1] = in ? *(const i32x4*)(row + ks + 64 + 16 * lg) : (i32x4){0, 0, 0, 0};
    }
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x5a5a5a5a) out[0] = 1;
}

}  // namespace

int main() {
  int dev = 0, cus = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  const int grid = cus;
  int* iout;
  float* fout;
  CHECK(hipMalloc(&iout, (size_t)grid * WG * sizeof(int)));
  CHECK(hipMalloc(&fout, (size_t)grid * WG * 4 * sizeof(float)));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  float ms = 0.f;

  std::printf("| probe | rate |\n|---|---:|\n");
  // LDS: 16 reads of 16 B per lane per iteration
  {
    const int iters = 20000;
    hipLaunchKernelGGL(k_lds, dim3(grid), dim3(WG), 0, 0, 100, iout);
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(k_lds, dim3(grid), dim3(WG), 0, 0, iters, iout);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    const double bytes = (double)grid * (WG / 64) * iters * 16 * 64 * 16;
    std::printf("| LDS 16-byte fragment reads, 8 waves/CU | %.1f TB/s (%.0f B per CU per ns) |\n",
                bytes / (ms * 1e-3) / 1e12, bytes / (ms * 1e-3) / 1e9 / grid);
  }
  // MFMA rates
  for (int scaled = 0; scaled < 2; ++scaled) {
    const int iters = 20000;
    auto launch = [&](int n) {
      if (scaled) hipLaunchKernelGGL(k_mfma<true>, dim3(grid), dim3(WG), 0, 0, n, fout);
      else hipLaunchKernelGGL(k_mfma<false>, dim3(grid), dim3(WG), 0, 0, n, fout);
    };
    launch(100);
    CHECK(hipEventRecord(e0));
    launch(iters);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    const double flops = (double)grid * (WG / 64) * iters * 16 * (16.0 * 16 * 128 * 2);
    std::printf("| FP8 MFMA 16x16x128, %s, 8 waves/CU | %.0f TFLOP/s |\n",
                scaled ? "block-scaled (zero-initialised product + one FMA per element)"
                       : "accumulated in place",
                flops / (ms * 1e-3) / 1e12);
  }
  // HBM reads
  {
    const size_t bytes = (size_t)2 * 2 * 14336 * 4096;   // 235 MB of weights
    const size_t flush = (size_t)1 << 30;
    uint8_t *w, *fl;
    CHECK(hipMalloc(&w, bytes));
    CHECK(hipMalloc(&fl, flush));
    CHECK(hipMemset(w, 1, bytes));
    CHECK(hipMemset(fl, 2, flush));
    auto timed = [&](auto launch, double nbytes, const char* name) -> int {
      float best = 1e30f;
      for (int rep = 0; rep < 5; ++rep) {
        hipLaunchKernelGGL(k_read_all, dim3(2048), dim3(256), 0, 0, (const i32x4*)fl, flush / 16, iout);
        CHECK(hipEventRecord(e0));
        launch();
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        best = ms < best ? ms : best;
      }
      std::printf("| %s | %.2f TB/s |\n", name, nbytes / (best * 1e-3) / 1e12);
      return 0;
    };
    if (timed([&] { hipLaunchKernelGGL(k_stream, dim3(4 * grid), dim3(256), 0, 0, (const i32x4*)w, bytes / 16, iout); },
              (double)bytes, "HBM read, contiguous non-temporal stream (235 MB)"))
      return 1;
    for (int K : {4096, 7168}) {
      const int rows = (int)(bytes / K) / 16 * 16;
      char name[128];
      std::snprintf(name, sizeof name, "HBM read, decode GEMM fragment pattern, K = %d (%.0f MB)", K, (double)rows * K / 1e6);
      if (timed([&] { hipLaunchKernelGGL(k_fragments, dim3(rows / 16), dim3(256), 0, 0, w, K, iout); },
                (double)rows * K, name))
        return 1;
    }
    CHECK(hipFree(w));
    CHECK(hipFree(fl));
  }
  CHECK(hipFree(iout));
  CHECK(hipFree(fout));
  return 0;
}
