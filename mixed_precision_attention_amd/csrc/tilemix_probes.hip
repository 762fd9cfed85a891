// Hardware-rate probes for gfx950 (MI355X): the measured rates behind the
// cost model of the attention kernels (vector-ALU issue, the matrix pipe
// beside the vector ALU, HBM->LDS copies, LDS reads, HBM read patterns of
// the decode step).  Timing-only kernels, built into their own library
// (libtilemix_probes.so) and run by the benchmark's probe leg; nothing of the
// attention path calls them.  Each kernel writes its result only when it
// equals a value it cannot take, so the work stays alive and the outputs
// stay untouched; every index stays inside the buffers whose sizes the entry
// points fix or check.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tilemix_probes.h"

namespace tilemix_probe {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int16v __attribute__((ext_vector_type(16)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short2v __attribute__((ext_vector_type(2)));

#define PROBE_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int kMagic = 0x2468ace1;

// --------------------------------------------------------------------------
// Vector-ALU issue: each thread runs 16 independent chains of one operation
// (0: fp32 FMA, 1: v_exp_f32); the grid sets the waves per SIMD (256 threads
// = one wave on each of a CU's 4 SIMDs).
// --------------------------------------------------------------------------
template <int OP>
__global__ __launch_bounds__(256) void valu_kernel(float* out, int iters, float c, float d) {
  constexpr int kChains = 16;
  float b[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) b[j] = 0.01f * j + 0.001f * (threadIdx.x & 63) - 0.5f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) {
      if constexpr (OP == 0) b[j] = __builtin_fmaf(b[j], c, d);
      else b[j] = __builtin_amdgcn_exp2f(-b[j]);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += b[j];
  if (__builtin_bit_cast(int, s) == kMagic) out[blockIdx.x * 256 + threadIdx.x] = s;
}

// --------------------------------------------------------------------------
// Matrix pipe beside the vector ALU: one 512-thread group per CU, waves 0-3
// (one per SIMD) run four independent 32x32x16 f16 MFMA chains, waves 4-7
// run eight FMA chains four times per iteration.  mode 1: matrix waves only,
// 2: vector waves only, 0: both.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(512) void coexec_kernel(float* out, int iters, int mode) {
  const int w = threadIdx.x >> 6;
  float r = 0.f;
  if (w < 4) {
    if (mode != 2) {
      half8 a, b;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(threadIdx.x * 0.001f + i);
        b[i] = (_Float16)(i * 0.5f);
      }
      float16v acc[4] = {};
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[k], 0, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int i = 0; i < 16; ++i) r += acc[k][i];
    }
  } else if (mode != 1) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = threadIdx.x * 1e-3f + j;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int rep = 0; rep < 4; ++rep)
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = __builtin_fmaf(x[j], 0.999f, 1e-4f);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) r += x[j];
  }
  if (__builtin_bit_cast(int, r) == kMagic) out[blockIdx.x * 512 + threadIdx.x] = r;
}

// --------------------------------------------------------------------------
// HBM/L2 -> LDS copy rate: a 512-thread group per CU with 128 KB of LDS;
// each wave issues `batch` direct 1 KB copies (buffer_load_dwordx4 ... lds)
// into its own 16 KB, waits for them, and repeats.  The source offsets walk
// a `src_kb` KB buffer (the buffer resource bounds every read).
// --------------------------------------------------------------------------
__global__ __launch_bounds__(512) void copy_kernel(const char* src, int src_kb, int iters, int batch, int* out) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const unsigned long long b = (unsigned long long)src;
  const int4v rsrc = {(int)__builtin_amdgcn_readfirstlane((unsigned)b),
                      (int)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32) & 0xffffu), src_kb * 1024, 0x00020000};
  const unsigned base =
      __builtin_amdgcn_readfirstlane((unsigned)(size_t)PROBE_LDS(char, lds)) + (unsigned)w * 16384u;
  int k = (blockIdx.x * 8 + w) * 37 % src_kb;
  for (int it = 0; it < iters; ++it) {
    for (int i = 0; i < batch; ++i) {
      k = (k + 1) % src_kb;
      const unsigned la = __builtin_amdgcn_readfirstlane(base + (unsigned)((i & 15) * 1024));
      const int soff = __builtin_amdgcn_readfirstlane(k * 1024);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(la),
                   "v"(lane * 16), "s"(rsrc), "s"(soff)
                   : "memory", "m0");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  const int v = lds[threadIdx.x * 16];
  if (v == kMagic) out[blockIdx.x * 512 + threadIdx.x] = v;
}

// --------------------------------------------------------------------------
// LDS read rate: a 512-thread group per CU, each wave reading its own 16 KB
// region, conflict-free, 16 KB per iteration: op 0 with ds_read_b128 (1 KB
// per instruction), op 1 with the transposing ds_read_b64_tr_b16 (512 B per
// instruction).
// --------------------------------------------------------------------------
template <int OP>
__global__ __launch_bounds__(512) void lds_kernel(int* out, int iters) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  char* region = lds + w * 16384;
  for (int i = lane; i < 16384 / 4; i += 64) reinterpret_cast<int*>(region)[i] = i * 2654435761u;
  __syncthreads();
  int x = 0;
  for (int it = 0; it < iters; ++it) {
    const int rot = (it & 15) * 16;
    if constexpr (OP == 0) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int off = (lane * 16 + j * 1024 + rot) & 16383;
        const int4v v = *PROBE_LDS(int4v, region + off);
        x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int off = (lane * 8 + j * 512 + rot) & 16383;
        const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(PROBE_LDS(short4v, region + off));
        x ^= __builtin_bit_cast(int, (short2v){v[0], v[1]}) ^ __builtin_bit_cast(int, (short2v){v[2], v[3]});
      }
    }
  }
  if (x == kMagic) out[blockIdx.x * 512 + threadIdx.x] = x;
}

// --------------------------------------------------------------------------
// HBM read patterns of the decode step over an int8 cache of kRows rows x
// kHeads heads x 128 bytes per operand (K and V, 32 MiB each), one
// 256-thread group per (256-row chunk, sequence of 4096 rows, head):
//   0: contiguous 64 KB per group (K then V as one span);
//   1: one 128-byte key row per lane (8 x 16 B), 4 bytes of value per lane
//      (32 lanes per row);
//   2: 8 lanes per key row (16 B each), values as in 1;
//   3: as 2 with the head fastest in the launch order.
// --------------------------------------------------------------------------
constexpr int kRows = TILEMIX_PROBE_READ_ROWS, kHeads = TILEMIX_PROBE_READ_HEADS, kD = 128;
constexpr int kGroups = (kRows / 256) * kHeads;  // 1024

template <int P>
__global__ __launch_bounds__(256) void read_kernel(const int8_t* K, const int8_t* V, int* out) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int x = 0;
  if constexpr (P == 0) {
    const int g = blockIdx.x;
    const int8_t* base = g < kGroups / 2 ? K + (size_t)g * 65536 : V + (size_t)(g - kGroups / 2) * 65536;
    int4v r[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = *reinterpret_cast<const int4v*>(base + i * 4096 + t * 16);
#pragma unroll
    for (int i = 0; i < 16; ++i) x ^= r[i][0] ^ r[i][1] ^ r[i][2] ^ r[i][3];
  } else {
    int c, s, kv;
    if constexpr (P == 3) {
      kv = blockIdx.x % kHeads;
      const int r = blockIdx.x / kHeads;
      c = r % 16;
      s = r / 16;
    } else {
      c = blockIdx.x % 16;
      const int sk = blockIdx.x / 16;
      s = sk / kHeads;
      kv = sk % kHeads;
    }
    const int row0 = s * 4096 + c * 256;
    int4v kr[8];
    if constexpr (P == 1) {
      const int8_t* krow = K + ((size_t)(row0 + w * 64 + lane) * kHeads + kv) * kD;
#pragma unroll
      for (int i = 0; i < 8; ++i) kr[i] = *reinterpret_cast<const int4v*>(krow + 16 * i);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        kr[i] = *reinterpret_cast<const int4v*>(K + ((size_t)(row0 + w * 64 + i * 8 + lane / 8) * kHeads + kv) * kD +
                                                (lane % 8) * 16);
    }
    const int c4 = t % 32, part = t / 32;
    int vr[32];
#pragma unroll
    for (int k = 0; k < 32; ++k)
      vr[k] = *reinterpret_cast<const int*>(V + ((size_t)(row0 + part * 32 + k) * kHeads + kv) * kD + c4 * 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) x ^= kr[i][0] ^ kr[i][1] ^ kr[i][2] ^ kr[i][3];
#pragma unroll
    for (int k = 0; k < 32; ++k) x ^= vr[k];
  }
  if (x == kMagic) out[blockIdx.x * 256 + t] = x;
}

// --------------------------------------------------------------------------
// Matrix skeleton of one prefill wave-tile, operands in registers (no loads):
// Q.K^T as 8 chained 32x32x32 int8 MFMAs (two 32-key blocks), the 32 int32
// scores per lane converted to fp32, EXTRA further FMAs spread over them,
// packed to fp16, then P.V as 16 32x32x16 f16 MFMAs into four accumulators.
// 768 matrix cycles per iteration at the published peak rates.
// --------------------------------------------------------------------------
template <int EXTRA>
__global__ __launch_bounds__(256) void skeleton_kernel(float* out, int iters, float c) {
  const int lane = threadIdx.x & 63;
  int4v kf[4], qb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kf[i] = (int4v){lane + i, 3 * lane + i, 5 * lane - i, 7 * lane} & 0x3f3f3f3f;
    qb[i] = (int4v){lane ^ i, lane * 11, i * 13, lane + 17} & 0x3f3f3f3f;
  }
  half8 vf[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 8; ++j) vf[db][j] = (_Float16)(0.001f * (lane + j + db));
  float16v o[4] = {};
  for (int it = 0; it < iters; ++it) {
    int16v acc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      acc[kb] = (int16v){};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[(kk + kb) & 3], qb[kk], acc[kb], 0, 0, 0);
    }
    float f[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      f[i] = (float)acc[0][i] * c;
      f[16 + i] = (float)acc[1][i] * c;
    }
#pragma unroll
    for (int e = 0; e < EXTRA; ++e) f[e & 31] = __builtin_fmaf(f[e & 31], c, 1e-3f);
    half8 pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[ks][j] = (_Float16)f[ks * 8 + j];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[db], pf[ks], o[db], 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) r += o[db][i];
  if (__builtin_bit_cast(int, r) == kMagic) out[blockIdx.x * 256 + threadIdx.x] = r;
}

// --------------------------------------------------------------------------
// Shader clock: every group runs FMA chains for `iters` steps; group 0's
// first wave stamps the shader-clock counter (s_memtime) and the 100 MHz
// real-time counter (s_memrealtime) before and after, out[0..3].
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void clock_kernel(long long* out, int iters) {
  const long long t0 = (long long)__builtin_amdgcn_s_memtime();
  const long long r0 = (long long)__builtin_amdgcn_s_memrealtime();
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = threadIdx.x * 1e-3f + j;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_fmaf(x[j], 0.999f, 1e-4f);
  }
  float r = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) r += x[j];
  const long long t1 = (long long)__builtin_amdgcn_s_memtime();
  const long long r1 = (long long)__builtin_amdgcn_s_memrealtime();
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    out[0] = t0;
    out[1] = t1;
    out[2] = r0;
    out[3] = __builtin_bit_cast(int, r) == kMagic ? 0 : r1;
  }
}

}  // namespace tilemix_probe

using namespace tilemix_probe;

extern "C" {

int tilemix_probe_valu(int op, int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (op) {
    case 0: hipLaunchKernelGGL(valu_kernel<0>, dim3(blocks), dim3(256), 0, st, out, iters, 0.999f, 0.001f); break;
    case 1: hipLaunchKernelGGL(valu_kernel<1>, dim3(blocks), dim3(256), 0, st, out, iters, 0.999f, 0.001f); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int tilemix_probe_coexec(int mode, int blocks, int iters, float* out, void* stream) {
  if (mode < 0 || mode > 2 || blocks <= 0 || iters <= 0 || out == nullptr) return -1;
  // 128 KB of (unused) LDS keeps it to one group per CU
  hipLaunchKernelGGL(coexec_kernel, dim3(blocks), dim3(512), 131072, static_cast<hipStream_t>(stream), out, iters,
                     mode);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int tilemix_probe_copy(const void* src, int src_kb, int blocks, int iters, int batch, int* out, void* stream) {
  if (src == nullptr || out == nullptr || src_kb <= 0 || src_kb > (1 << 20) || blocks <= 0 || iters <= 0 ||
      batch <= 0 || batch > 16)
    return -1;
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(512), 131072, static_cast<hipStream_t>(stream),
                     static_cast<const char*>(src), src_kb, iters, batch, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int tilemix_probe_lds(int op, int blocks, int iters, int* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (op == 0) hipLaunchKernelGGL(lds_kernel<0>, dim3(blocks), dim3(512), 131072, st, out, iters);
  else if (op == 1) hipLaunchKernelGGL(lds_kernel<1>, dim3(blocks), dim3(512), 131072, st, out, iters);
  else return -1;
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int tilemix_probe_skeleton(int extra, int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (extra) {
    case 0: hipLaunchKernelGGL(skeleton_kernel<0>, dim3(blocks), dim3(256), 0, st, out, iters, 1e-6f); break;
    case 64: hipLaunchKernelGGL(skeleton_kernel<64>, dim3(blocks), dim3(256), 0, st, out, iters, 1e-6f); break;
    case 128: hipLaunchKernelGGL(skeleton_kernel<128>, dim3(blocks), dim3(256), 0, st, out, iters, 1e-6f); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int tilemix_probe_clock(int blocks, int iters, long long* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return -1;
  hipLaunchKernelGGL(clock_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int tilemix_probe_read(int pattern, const void* k, const void* v, int* out, void* stream) {
  if (k == nullptr || v == nullptr || out == nullptr) return -1;
  const int8_t* kk = static_cast<const int8_t*>(k);
  const int8_t* vv = static_cast<const int8_t*>(v);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(kGroups), block(256);
  switch (pattern) {
    case 0: hipLaunchKernelGGL(read_kernel<0>, grid, block, 0, st, kk, vv, out); break;
    case 1: hipLaunchKernelGGL(read_kernel<1>, grid, block, 0, st, kk, vv, out); break;
    case 2: hipLaunchKernelGGL(read_kernel<2>, grid, block, 0, st, kk, vv, out); break;
    case 3: hipLaunchKernelGGL(read_kernel<3>, grid, block, 0, st, kk, vv, out); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
