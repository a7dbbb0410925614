// Measurement probes, not part of the AdaHOP path: the steady-state rate and
// shader clock of the FP4 matrix cores with no memory traffic, the practical
// ceiling any FP4 GEMM on this device runs under, and the LDS read bandwidth
// per CU.
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

}  // extern "C"
