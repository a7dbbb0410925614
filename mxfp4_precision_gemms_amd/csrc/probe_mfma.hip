// Measurement probes, not part of the AdaHOP path: the steady-state rate and
// shader clock of the FP4 matrix cores with no memory traffic, the practical
// ceiling any FP4 GEMM on this device runs under; the LDS read bandwidth per
// CU; and the HBM streaming rates (read, write, copy; ordinary and
// non-temporal loads; the 32-row block pattern of the column-direction
// quantizer) that bound the memory-bound kernels.
//
// One 512-thread workgroup per CU keeps 8 independent 32x32x64 scaled FP4
// MFMAs per wave in flight on register operands that differ per lane and per
// MFMA (pseudo-random E2M1 codes), so the multipliers switch as they do on
// real data; constant operands draw less power and let the clock run higher.
// The shader clock over the loop is s_memtime (shader clock cycles) against
// s_memrealtime (a 100 MHz counter).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

struct ProbeOut {
  unsigned long long cycles, realtime;
};

__global__ void __launch_bounds__(512) mfma_fp4_probe_kernel(ProbeOut* out, int iters, float* sink) {
  const int tid = threadIdx.x;
  v16f acc[8];
  for (int a = 0; a < 8; ++a)
    for (int v = 0; v < 16; ++v) acc[a][v] = 0.0f;
  v4i fa[4], fb[2];
  unsigned h = 0x9E3779B9u * (unsigned)(tid + 1 + 512 * blockIdx.x);
  auto next = [&]() { h ^= h << 13; h ^= h >> 17; h ^= h << 5; return (int)(h & 0x77777777u); };
  for (int i = 0; i < 4; ++i)
    for (int e = 0; e < 4; ++e) fa[i][e] = next();
  for (int i = 0; i < 2; ++i)
    for (int e = 0; e < 4; ++e) fb[i][e] = next();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[2 * i + j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            v8i{fb[j][0], fb[j][1], fb[j][2], fb[j][3], 0, 0, 0, 0},
            v8i{fa[i][0], fa[i][1], fa[i][2], fa[i][3], 0, 0, 0, 0}, acc[2 * i + j], 4, 4, 0, 127, 0, 127);
  }
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (tid == 0) {
    out[blockIdx.x].cycles = t1 - t0;
    out[blockIdx.x].realtime = r1 - r0;
  }
  float s = 0.0f;
  for (int a = 0; a < 8; ++a) s += acc[a][0];
  if (s == 1234.5f) sink[tid] = s;   // keeps the MFMAs live; never true for these codes' sums
}

// The same with 16x16x128 scaled FP4 MFMAs: 16 independent blocks per wave
// (the same 128 x 64 outputs per wave, half the accumulator bytes per MAC).
__global__ void __launch_bounds__(512) mfma_fp4_16_probe_kernel(ProbeOut* out, int iters, float* sink) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x;
  v4f acc[16];
  for (int a = 0; a < 16; ++a)
    for (int v = 0; v < 4; ++v) acc[a][v] = 0.0f;
  v4i fa[4], fb[4];
  unsigned h = 0x9E3779B9u * (unsigned)(tid + 1 + 512 * blockIdx.x);
  auto next = [&]() { h ^= h << 13; h ^= h >> 17; h ^= h << 5; return (int)(h & 0x77777777u); };
  for (int i = 0; i < 4; ++i)
    for (int e = 0; e < 4; ++e) fa[i][e] = next();
  for (int i = 0; i < 4; ++i)
    for (int e = 0; e < 4; ++e) fb[i][e] = next();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[4 * i + j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            v8i{fb[j][0], fb[j][1], fb[j][2], fb[j][3], 0, 0, 0, 0},
            v8i{fa[i][0], fa[i][1], fa[i][2], fa[i][3], 0, 0, 0, 0}, acc[4 * i + j], 4, 4, 0, 127, 0, 127);
  }
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (tid == 0) {
    out[blockIdx.x].cycles = t1 - t0;
    out[blockIdx.x].realtime = r1 - r0;
  }
  float s = 0.0f;
  for (int a = 0; a < 16; ++a) s += acc[a][0];
  if (s == 1234.5f) sink[tid] = s;   // keeps the MFMAs live; never true for these codes' sums
}

// 16x16x128 scaled FP4 MFMAs with one wave per SIMD (a 256-thread workgroup
// per CU): 64 independent blocks per wave (128 x 128 outputs, the
// accumulators in the 256 AGPRs the single wave may hold), the layout that
// would read each fragment from LDS once per 8 MFMAs instead of once per 2.
// Lds: the fragments of the next iteration (8 A and 8 B, 16 bytes per lane
// each) are read from a 64 KB LDS array during this iteration's MFMAs, as a
// GEMM would; else they stay in registers.
template <bool Lds>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_fp4_16_w1_probe_kernel(ProbeOut* out, int iters, float* sink) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  __shared__ uint4 lds[4096];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned h = 0x9E3779B9u * (unsigned)(tid + 1 + 256 * blockIdx.x);
  auto next = [&]() { h ^= h << 13; h ^= h >> 17; h ^= h << 5; return h & 0x77777777u; };
  for (int i = tid; i < 4096; i += 256) lds[i] = make_uint4(next(), next(), next(), next());
  __syncthreads();
  v4f acc[64];
#pragma unroll
  for (int a = 0; a < 64; ++a) acc[a] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  v4i fa0[8], fb0[8], fa1[8], fb1[8];
  // Fragment f of iteration it: 16 bytes per lane, consecutive lanes 16
  // bytes apart (no bank conflicts), always inside the array.
  auto rd = [&](int it, int f) {
    const uint4 q = lds[(f * 256 + wave * 64 + lane + it * 7) & 4095];
    return v4i{(int)q.x, (int)q.y, (int)q.z, (int)q.w};
  };
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    fa0[f] = rd(0, f);
    fb0[f] = rd(0, 8 + f);
    fa1[f] = fa0[f];
    fb1[f] = fb0[f];
  }
  auto mm = [&](v4i (&fa)[8], v4i (&fb)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[8 * i + j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            v8i{fb[j][0], fb[j][1], fb[j][2], fb[j][3], 0, 0, 0, 0},
            v8i{fa[i][0], fa[i][1], fa[i][2], fa[i][3], 0, 0, 0, 0}, acc[8 * i + j], 4, 4, 0, 127, 0, 127);
  };
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it += 2) {
    if (Lds) {
#pragma unroll
      for (int f = 0; f < 8; ++f) { fa1[f] = rd(it + 1, f); fb1[f] = rd(it + 1, 8 + f); }
    }
    mm(fa0, fb0);
    if (Lds) {
#pragma unroll
      for (int f = 0; f < 8; ++f) { fa0[f] = rd(it + 2, f); fb0[f] = rd(it + 2, 8 + f); }
    }
    mm(fa1, fb1);
  }
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (tid == 0) {
    out[blockIdx.x].cycles = t1 - t0;
    out[blockIdx.x].realtime = r1 - r0;
  }
  float s = 0.0f;
#pragma unroll
  for (int a = 0; a < 64; ++a) s += acc[a][0];
  if (s == 1234.5f) sink[tid] = s;   // keeps the MFMAs live; never true for these codes' sums
}

// LDS read bandwidth: every thread of a 512-thread workgroup reads 16-byte
// chunks, consecutive lanes 16 bytes apart (no bank conflicts), 8 reads per
// iteration, from a 128 KB array.
__global__ void __launch_bounds__(512) lds_read_probe_kernel(ProbeOut* out, int iters, unsigned* sink) {
  __shared__ __attribute__((aligned(16))) uint4 buf[8192];
  const int tid = threadIdx.x;
  for (int i = tid; i < 8192; i += 512) buf[i] = make_uint4(i, 3 * i, 5 * i, 7 * i);
  __syncthreads();
  unsigned acc = 0;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    const int base = (it * 64) & 4095;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 q = buf[(base + tid + j * 512) & 8191];
      acc ^= q.x + q.y + q.z + q.w;
    }
  }
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (tid == 0) {
    out[blockIdx.x].cycles = t1 - t0;
    out[blockIdx.x].realtime = r1 - r0;
  }
  if (acc == 0x12345678u) sink[tid] = acc;
}

template <typename Launch>
int run_probe(Launch launch, int blocks, int launches, void* scratch, double* cycles, double* ticks) {
  ProbeOut* out = static_cast<ProbeOut*>(scratch);
  ProbeOut* host = new ProbeOut[blocks];
  int rc = 0;
  for (int l = 0; l < launches && rc == 0; ++l) {
    launch(out, reinterpret_cast<char*>(scratch) + (size_t)blocks * sizeof(ProbeOut));
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpy(host, out, (size_t)blocks * sizeof(ProbeOut), hipMemcpyDeviceToHost);
    if (e != hipSuccess) { rc = (int)e; break; }
    double c = 0, t = 0;
    for (int b = 0; b < blocks; ++b) { c += (double)host[b].cycles; t += (double)host[b].realtime; }
    cycles[l] = c / blocks;
    ticks[l] = t / blocks;
  }
  delete[] host;
  return rc;
}

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Streaming kernels over n 16-byte words, 256 threads, U independent words
// per thread per step, grid-stride; every index stays below n.
template <bool NT>
__global__ void __launch_bounds__(256) stream_read_kernel(const v4u* __restrict__ p, size_t n,
                                                          unsigned* sink) {
  constexpr int U = 8;
  size_t i = (size_t)blockIdx.x * 256 * U + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256 * U;
  unsigned acc = 0;
  for (; i + 256 * (U - 1) < n; i += stride) {
    v4u v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(p + i + 256 * u) : p[i + 256 * u];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x12345678u) sink[threadIdx.x] = acc;
}

__global__ void __launch_bounds__(256) stream_write_kernel(v4u* __restrict__ p, size_t n) {
  constexpr int U = 4;
  size_t i = (size_t)blockIdx.x * 256 * U + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256 * U;
  for (; i + 256 * (U - 1) < n; i += stride) {
#pragma unroll
    for (int u = 0; u < U; ++u) p[i + 256 * u] = v4u{(unsigned)i, 1u, 2u, 3u};
  }
}

template <bool NT>
__global__ void __launch_bounds__(256) stream_copy_kernel(const v4u* __restrict__ s, v4u* __restrict__ d,
                                                          size_t n) {
  constexpr int U = 4;
  size_t i = (size_t)blockIdx.x * 256 * U + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256 * U;
  for (; i + 256 * (U - 1) < n; i += stride) {
    v4u v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(s + i + 256 * u) : s[i + 256 * u];
#pragma unroll
    for (int u = 0; u < U; ++u) d[i + 256 * u] = v[u];
  }
}

// The column-direction quantizer's read pattern over a [rows][ldb bytes]
// matrix: workgroup (x, y) covers 512 bytes of columns and 128 rows; wave w
// reads 32 rows of its 32-row block, 8 bytes per lane per row, at scalar row
// offsets of one buffer descriptor. Cache policy AUX (2 = non-temporal).
template <int AUX>
__global__ void __launch_bounds__(256) colblock_read_kernel(const uint8_t* __restrict__ p, int64_t rows,
                                                            int64_t ldb, unsigned* sink) {
  const int tid = threadIdx.x, cg = tid % 64, bi = tid / 64;
  const int64_t col = (int64_t)blockIdx.x * 512 + 8 * cg;
  const int64_t r0 = ((int64_t)blockIdx.y * 4 + bi) * 32;
  if (r0 + 32 > rows || col + 8 > ldb) return;
  const uint8_t* blk = p + (int64_t)blockIdx.y * 128 * ldb;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blk), 0, 0x7FFFFFFF, 0x00020000);
  const int voff = (int)(bi * 32 * ldb + col);
  unsigned acc = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const auto q = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, (int)(j * ldb), AUX);
    acc ^= q[0] ^ q[1];
  }
  if (acc == 0x12345678u) sink[tid] = acc;
}

template <typename Launch>
int time_launches(Launch launch, int launches, float* ms) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  for (int l = 0; l < launches && e == hipSuccess; ++l) {
    e = hipEventRecord(e0, 0);
    if (e == hipSuccess) launch();
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) e = hipEventRecord(e1, 0);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms[l], e0, e1);
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  return (int)e;
}

}  // namespace

extern "C" {

// Runs `launches` launches of `blocks` workgroups, each `iters` iterations of
// 8 MFMAs per wave, back to back, and writes per launch the mean shader-clock
// cycles and 100 MHz ticks over the MFMA loop (host arrays of `launches`).
// `scratch` is a caller device buffer of blocks * 16 + 2048 bytes.
// Returns 0, or the hipError_t of the first failing call.
__attribute__((visibility("default"))) int adahop_probe_mfma_fp4(int blocks, int iters, int launches,
                                                                 void* scratch, double* cycles,
                                                                 double* ticks) {
  if (blocks < 1 || iters < 1 || launches < 1 || !scratch || !cycles || !ticks)
    return (int)hipErrorInvalidValue;
  return run_probe([&](ProbeOut* out, char* sink) {
    mfma_fp4_probe_kernel<<<dim3(blocks), dim3(512)>>>(out, iters, reinterpret_cast<float*>(sink));
  }, blocks, launches, scratch, cycles, ticks);
}

// As adahop_probe_mfma_fp4 with 16x16x128 MFMAs: 16 per wave per iteration
// (the same multiply-adds as the 8 32x32x64 ones).
__attribute__((visibility("default"))) int adahop_probe_mfma_fp4_16(int blocks, int iters, int launches,
                                                                    void* scratch, double* cycles,
                                                                    double* ticks) {
  if (blocks < 1 || iters < 1 || launches < 1 || !scratch || !cycles || !ticks)
    return (int)hipErrorInvalidValue;
  return run_probe([&](ProbeOut* out, char* sink) {
    mfma_fp4_16_probe_kernel<<<dim3(blocks), dim3(512)>>>(out, iters, reinterpret_cast<float*>(sink));
  }, blocks, launches, scratch, cycles, ticks);
}

// As adahop_probe_mfma_fp4 with one wave per SIMD (256-thread workgroups), 64
// 16x16x128 MFMAs per wave per iteration, the fragments read from LDS
// (lds != 0) or kept in registers; iters even.
__attribute__((visibility("default"))) int adahop_probe_mfma_fp4_16_w1(int lds, int blocks, int iters,
                                                                       int launches, void* scratch,
                                                                       double* cycles, double* ticks) {
  if (blocks < 1 || iters < 2 || iters % 2 != 0 || launches < 1 || !scratch || !cycles || !ticks)
    return (int)hipErrorInvalidValue;
  return run_probe([&](ProbeOut* out, char* sink) {
    if (lds)
      mfma_fp4_16_w1_probe_kernel<true><<<dim3(blocks), dim3(256)>>>(out, iters, reinterpret_cast<float*>(sink));
    else
      mfma_fp4_16_w1_probe_kernel<false><<<dim3(blocks), dim3(256)>>>(out, iters, reinterpret_cast<float*>(sink));
  }, blocks, launches, scratch, cycles, ticks);
}

// As adahop_probe_mfma_fp4 for the LDS read probe: each workgroup reads
// 8 x 512 x 16 bytes per iteration.
__attribute__((visibility("default"))) int adahop_probe_lds_read(int blocks, int iters, int launches,
                                                                 void* scratch, double* cycles,
                                                                 double* ticks) {
  if (blocks < 1 || iters < 1 || launches < 1 || !scratch || !cycles || !ticks)
    return (int)hipErrorInvalidValue;
  return run_probe([&](ProbeOut* out, char* sink) {
    lds_read_probe_kernel<<<dim3(blocks), dim3(512)>>>(out, iters, reinterpret_cast<unsigned*>(sink));
  }, blocks, launches, scratch, cycles, ticks);
}

// HBM streaming rates on the null stream: mode 0 reads `a` (nt: with
// non-temporal loads), 1 writes `a`, 2 copies `a` to `b` (nt: non-temporal
// loads), 3 reads `a` as the column-direction quantizer does, as a
// [rows = bytes / 28672][28672 bytes] matrix (nt: cache policy NT).
// `bytes` is a multiple of 16 (of 28672 for mode 3), `a` and `b` device
// buffers of `bytes` (b unused except in mode 2), `sink` a device buffer of
// 1 KB; `grid` workgroups of 256 threads (modes 0-2). Writes the duration of
// each of `launches` launches in ms to the host array `ms`. Returns 0, or the
// hipError_t of the first failing call.
__attribute__((visibility("default"))) int adahop_probe_hbm(int mode, int nt, void* a, void* b,
                                                            size_t bytes, int grid, int launches,
                                                            void* sink, float* ms) {
  if (mode < 0 || mode > 3 || !a || (mode == 2 && !b) || !sink || !ms || launches < 1 ||
      bytes < 16 || bytes % 16 != 0 || grid < 1)
    return (int)hipErrorInvalidValue;
  const size_t n = bytes / 16;
  v4u* pa = static_cast<v4u*>(a);
  v4u* pb = static_cast<v4u*>(b);
  unsigned* sk = static_cast<unsigned*>(sink);
  switch (mode) {
    case 0:
      return time_launches([&] {
        if (nt) stream_read_kernel<true><<<dim3(grid), dim3(256)>>>(pa, n, sk);
        else stream_read_kernel<false><<<dim3(grid), dim3(256)>>>(pa, n, sk);
      }, launches, ms);
    case 1:
      return time_launches([&] { stream_write_kernel<<<dim3(grid), dim3(256)>>>(pa, n); }, launches, ms);
    case 2:
      return time_launches([&] {
        if (nt) stream_copy_kernel<true><<<dim3(grid), dim3(256)>>>(pa, pb, n);
        else stream_copy_kernel<false><<<dim3(grid), dim3(256)>>>(pa, pb, n);
      }, launches, ms);
    default: {
      const int64_t ldb = 28672, rows = (int64_t)(bytes / ldb) / 128 * 128;
      if (rows < 128 || (int64_t)bytes < rows * ldb) return (int)hipErrorInvalidValue;
      const dim3 g((unsigned)(ldb / 512), (unsigned)(rows / 128));
      const uint8_t* p = static_cast<const uint8_t*>(a);
      return time_launches([&] {
        if (nt) colblock_read_kernel<2><<<g, dim3(256)>>>(p, rows, ldb, sk);
        else colblock_read_kernel<0><<<g, dim3(256)>>>(p, rows, ldb, sk);
      }, launches, ms);
    }
  }
}

}  // extern "C"
