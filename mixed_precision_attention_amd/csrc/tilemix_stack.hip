// Device half of the synthetic multi-layer stack for gfx950: RMS norm,
// grouped projections on the f16 matrix cores, and one whole layer (norm,
// Q/K/V projection, blockwise quantisation, TileMix prefill, output
// projection with the residual add).
//
// Source (web page about TileMix, cited by title and section):
//   [Explainer] "TileMix：给AI大模型的“注意力”做一次精准的精度分配手术",
//               section 数字精度混用到底靠不靠谱 (deeper models accumulate more
//               deviation, the error of a layer being carried into the next).
//   [Digest]    "TileMix: Tile-Centric Mixed-Precision Attention for LLM
//               Inference Acceleration", method paragraph (FP16 attention
//               operands; one static template reused across layers).
//
// The pages describe no layer beyond attention.  The stack keeps what carries
// an error from one layer to the next: attention whose Q, K and V are
// computed from the running hidden state, and a residual connection.  The
// hidden state x [T, Hq*d] (fp32) splits into Hkv independent streams of
// width W = (Hq/Hkv)*d -- stream g is channels g*W .. g*W+W-1, owned by KV
// head g and its query heads -- and a layer is, per stream,
//   u = x_g / sqrt(mean(x_g^2) + eps)              (fp16)
//   [q | k | v] = u . Wqkv_g^T                      (fp16, Wqkv_g (W+2d) x W)
//   o = TileMix prefill attention of (q, k, v)      (fp16)
//   x_g += o_g . Wo_g^T                             (fp32, Wo_g W x W)
// Row n < W of Wqkv_g feeds query head g*Hq/Hkv + n/d, channel n % d; rows
// W .. W+d-1 feed K of KV head g, the last d rows its V.
//
// gfx950 matrix instruction used (lane l of a 64-wide wave, c = l % 32,
// hh = l / 32): v_mfma_f32_32x32x16_f16 takes A[c][hh*8 + j] and
// B[hh*8 + j][c], j = 0..7, and leaves accumulator element i (0..15) at
// C[(i/4)*8 + hh*4 + i%4][c].

#include <hip/hip_runtime.h>

#include "tilemix.h"
#include "tilemix_host.h"
#include "tilemix_internal.h"

namespace tilemix {
namespace stack {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves of 64
constexpr int kMaxPerLane = 16;  // W <= 1024 channels per stream

// --------------------------------------------------------------------------
// RMS norm.  One wave per (token, stream) row of W channels: x viewed as
// [T*Hkv][W] since Hq*d = Hkv*W; each lane holds kVec-wide pieces (kVec = 4,
// 2 or 1 as W allows) in registers.  Sum of squares in fp32, then
// u = fl16(x * fl32(1 / sqrt(fl32(ss / W) + eps))).
// --------------------------------------------------------------------------
struct NormArgs {
  const float* x;
  _Float16* u;
  int64_t rows;  // T * Hkv
  int32_t W;
  float eps;
};

template <int kVec>
__global__ __launch_bounds__(kThreads) void rms_norm_kernel(NormArgs a) {
  typedef float floatv __attribute__((ext_vector_type(kVec)));
  typedef _Float16 halfv __attribute__((ext_vector_type(kVec)));
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const floatv* xr = reinterpret_cast<const floatv*>(a.x + row * a.W);
  halfv* ur = reinterpret_cast<halfv*>(a.u + row * a.W);
  const int n = a.W / (64 * kVec);
  floatv v[kMaxPerLane / kVec];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxPerLane / kVec; ++i) {
    if (i < n) {
      v[i] = xr[lane + 64 * i];
#pragma unroll
      for (int j = 0; j < kVec; ++j) ss = fmaf(v[i][j], v[i][j], ss);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float inv = __fdiv_rn(1.0f, __fsqrt_rn(__fdiv_rn(ss, (float)a.W) + a.eps));
#pragma unroll
  for (int i = 0; i < kMaxPerLane / kVec; ++i) {
    if (i < n) {
      halfv h;
#pragma unroll
      for (int j = 0; j < kVec; ++j) h[j] = (_Float16)(v[i][j] * inv);
      ur[lane + 64 * i] = h;
    }
  }
}

// --------------------------------------------------------------------------
// Grouped projection C = A_g . B_g^T on the f16 matrix cores, fp32
// accumulation.  A_g: the stream-g slice of T rows of width W (row stride
// Hq*d halves); B_g: N rows of W halves (row n = the weights of output n).
// Workgroup tile 128 tokens x 128 outputs; the W-long reduction runs in
// 64-wide chunks staged through LDS (rows padded to 144 bytes, so the
// 16-byte fragment reads of 8 consecutive lanes hit distinct banks); the next
// chunk's global loads are in flight while the current one is multiplied.
// Wave (wm, wn) computes the 64 x 64 sub-tile at (64 wm, 64 wn).
// Epilogue: either Q/K/V in fp16 (kResidual = false) or x += C in fp32.
// --------------------------------------------------------------------------
constexpr int kTileM = 128;
constexpr int kTileN = 128;
constexpr int kTileK = 64;
constexpr int kPitch = 144;
constexpr int kTileBytes = kTileM * kPitch;

struct ProjArgs {
  const _Float16* a;  // [T, Hq*d]
  const _Float16* w;  // [Hkv, N, W]
  _Float16* q;        // [T, Hq, d]
  _Float16* k;        // [T, Hkv, d]
  _Float16* v;        // [T, Hkv, d]
  float* x;           // [T, Hq*d]
  int64_t T;
  int32_t W, N, d, hq, hkv;
  int32_t col_tiles, row_tiles, units;  // units = Hkv * row_tiles * col_tiles
};

constexpr int kDies = 8;  // XCDs of an MI355X; workgroups are dealt round-robin

template <bool kResidual>
__global__ __launch_bounds__(kThreads, 4) void proj_kernel(ProjArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kTileBytes];
  char* sA = smem;
  char* sB = smem + kTileBytes;
  // XCD-aware order: workgroup i runs on die i % 8, so unit
  // u = (i % 8) * per_die + i / 8 gives each die a contiguous run of units,
  // column tiles fastest: the column tiles that share a token tile's A rows
  // meet in one die's L2, and a die works through few streams' weights.
  const int64_t per_die = ((int64_t)p.units + kDies - 1) / kDies;
  const int64_t u = (int64_t)(blockIdx.x % kDies) * per_die + blockIdx.x / kDies;
  if (u >= p.units) return;  // before any barrier
  const int n0 = (int)(u % p.col_tiles) * kTileN;
  const int64_t m0 = ((u / p.col_tiles) % p.row_tiles) * kTileM;
  const int g = (int)(u / ((int64_t)p.col_tiles * p.row_tiles));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int c = lane & 31, hh = lane >> 5;
  const int64_t lda = (int64_t)p.hq * p.d;

  // Global -> LDS copy: thread tid moves 16 bytes (segment tid % 8) of rows
  // tid / 8 + 32 j, j = 0..3, of both tiles.  Rows past the end repeat the
  // last row (their results are not stored).
  // Addresses: a wave-uniform base per tile plus 32-bit lane offsets (the
  // tile spans at most 128 rows), which keeps the copy's address registers
  // few enough for four workgroups per CU.
  const int lr = tid >> 3, ls = tid & 7;
  const _Float16* abase = p.a + m0 * lda + (int64_t)g * p.W;
  const _Float16* bbase = p.w + ((int64_t)g * p.N + n0) * p.W;
  uint32_t oa[4], ob[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t t = min(m0 + lr + 32 * j, p.T - 1) - m0;
    oa[j] = (uint32_t)(t * lda) + ls * 8;
    const int n = min(n0 + lr + 32 * j, p.N - 1) - n0;
    ob[j] = (uint32_t)(n * p.W) + ls * 8;
  }
  int4v ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ra[j] = *reinterpret_cast<const int4v*>(abase + oa[j] + k0);
      rb[j] = *reinterpret_cast<const int4v*>(bbase + ob[j] + k0);
    }
  };

  float16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (float16v){};

  const int nk = p.W / kTileK;
  gload(0);
  for (int kc = 0; kc < nk; ++kc) {
    __syncthreads();  // the previous chunk's fragments have been read
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<int4v*>(sA + (lr + 32 * j) * kPitch + ls * 16) = ra[j];
      *reinterpret_cast<int4v*>(sB + (lr + 32 * j) * kPitch + ls * 16) = rb[j];
    }
    __syncthreads();
    if (kc + 1 < nk) gload((kc + 1) * kTileK);
#pragma unroll
    for (int kk = 0; kk < kTileK / 16; ++kk) {
      half8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const half8*>(sA + (wm * 64 + i * 32 + c) * kPitch + kk * 32 + hh * 16);
        bf[i] = *reinterpret_cast<const half8*>(sB + (wn * 64 + i * 32 + c) * kPitch + kk * 32 + hh * 16);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue.  Each wave's 64 x 64 block goes out in two halves of 32 rows:
  // the accumulators are written to a wave-private LDS area (rows of 72
  // floats, so the two half-waves, 4 rows apart, hit disjoint banks), then
  // read back as 16-byte row pieces and stored (fp16 Q/K/V) or added to x
  // (fp32) with full vectors, all of a lane's loads in flight together.
  // N, W and d are multiples of 64, so a wave's 64 columns lie in one of
  // q, k, v and either all or none of them exist.
  __syncthreads();  // every wave is done with the operand tiles
  const int nb = n0 + wn * 64;
  if (nb >= p.N) return;  // no barrier follows
  constexpr int kRow = 72;
  float* sC = reinterpret_cast<float*>(smem) + wave * (32 * kRow);
  int64_t stride;
  char* dst;
  if (kResidual) {
    stride = lda * 4;
    dst = reinterpret_cast<char*>(p.x + (int64_t)g * p.W + nb);
  } else if (nb < p.W) {
    stride = lda * 2;
    dst = reinterpret_cast<char*>(p.q + (int64_t)g * p.W + nb);
  } else if (nb < p.W + p.d) {
    stride = (int64_t)p.hkv * p.d * 2;
    dst = reinterpret_cast<char*>(p.k + (int64_t)g * p.d + (nb - p.W));
  } else {
    stride = (int64_t)p.hkv * p.d * 2;
    dst = reinterpret_cast<char*>(p.v + (int64_t)g * p.d + (nb - p.W - p.d));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) sC[((e >> 2) * 8 + hh * 4 + (e & 3)) * kRow + j * 32 + c] = acc[i][j][e];
    __builtin_amdgcn_wave_barrier();
    const int64_t r0 = m0 + wm * 64 + i * 32;
    // 32 rows x 16 float4: lane handles piece lane + 64 s -> row 4 s + lane / 16,
    // column 4 (lane % 16); four pieces per batch
    const int col4 = (lane & 15) * 4;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float4 part[4];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int row = 4 * (4 * b + s4) + (lane >> 4);
        part[s4] = *reinterpret_cast<const float4*>(sC + row * kRow + col4);
      }
      if (kResidual) {
        float4 xv[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int64_t t = r0 + 4 * (4 * b + s4) + (lane >> 4);
          if (t < p.T) xv[s4] = *reinterpret_cast<const float4*>(dst + t * stride + col4 * 4);
        }
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int64_t t = r0 + 4 * (4 * b + s4) + (lane >> 4);
          if (t < p.T) {
            const float4 o = {xv[s4].x + part[s4].x, xv[s4].y + part[s4].y, xv[s4].z + part[s4].z,
                              xv[s4].w + part[s4].w};
            *reinterpret_cast<float4*>(dst + t * stride + col4 * 4) = o;
          }
        }
      } else {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int64_t t = r0 + 4 * (4 * b + s4) + (lane >> 4);
          if (t < p.T) {
            typedef _Float16 half4v __attribute__((ext_vector_type(4)));
            const half4v h = {(_Float16)part[s4].x, (_Float16)part[s4].y, (_Float16)part[s4].z,
                              (_Float16)part[s4].w};
            *reinterpret_cast<half4v*>(dst + t * stride + col4 * 2) = h;
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();  // the second half reuses the area
  }
}

// --------------------------------------------------------------------------
// Host side
// --------------------------------------------------------------------------
namespace {

int hip_fail(hipError_t e, const char* what) {
  return fail(TILEMIX_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int check_ptr(const void* p, const char* name, bool needed) {
  if (!needed) return TILEMIX_OK;
  if (p == nullptr) return fail(TILEMIX_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(TILEMIX_EINVAL, "%s is not 16-byte aligned", name);
  return TILEMIX_OK;
}

int check_shape(int64_t tokens, int32_t hq, int32_t hkv, int32_t d) {
  if (tokens < 0) return fail(TILEMIX_EINVAL, "tokens = %lld is negative", (long long)tokens);
  if (d != 64 && d != 128) return fail(TILEMIX_EUNSUPPORTED, "head_dim %d (64 or 128)", d);
  if (hkv < 1 || hq < 1 || hq % hkv) return fail(TILEMIX_EINVAL, "Hq = %d is not a multiple of Hkv = %d", hq, hkv);
  if ((int64_t)(hq / hkv) * d > 64 * kMaxPerLane)
    return fail(TILEMIX_EUNSUPPORTED, "stream width (Hq/Hkv)*d = %d exceeds %d", (hq / hkv) * d, 64 * kMaxPerLane);
  if (hkv > 65535) return fail(TILEMIX_EINVAL, "Hkv = %d too large for one launch", hkv);
  if ((tokens + kTileM - 1) / kTileM > 65535) return fail(TILEMIX_EINVAL, "too many tokens for one launch");
  return TILEMIX_OK;
}

int launch_norm(const float* x, _Float16* u, int64_t tokens, int32_t hq, int32_t hkv, int32_t d, float eps,
                hipStream_t st) {
  NormArgs a;
  a.x = x;
  a.u = u;
  a.rows = tokens * hkv;
  a.W = (hq / hkv) * d;
  a.eps = eps;
  const int64_t blocks = (a.rows + 3) / 4;
  if (blocks > 0x7fffffff) return fail(TILEMIX_EINVAL, "too many tokens for one launch");
  if (a.W % 256 == 0)
    hipLaunchKernelGGL(rms_norm_kernel<4>, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  else if (a.W % 128 == 0)
    hipLaunchKernelGGL(rms_norm_kernel<2>, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(rms_norm_kernel<1>, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TILEMIX_OK : hip_fail(e, "rms norm launch");
}

int launch_proj(bool residual, const _Float16* a_in, const _Float16* w, _Float16* q, _Float16* k, _Float16* v,
                float* x, int64_t tokens, int32_t hq, int32_t hkv, int32_t d, hipStream_t st) {
  ProjArgs p;
  p.a = a_in;
  p.w = w;
  p.q = q;
  p.k = k;
  p.v = v;
  p.x = x;
  p.T = tokens;
  p.W = (hq / hkv) * d;
  p.N = residual ? p.W : p.W + 2 * d;
  p.d = d;
  p.hq = hq;
  p.hkv = hkv;
  p.col_tiles = (p.N + kTileN - 1) / kTileN;
  p.row_tiles = (int32_t)((tokens + kTileM - 1) / kTileM);
  const int64_t units = (int64_t)hkv * p.row_tiles * p.col_tiles;
  if (units > 0x7fffffff - kDies) return fail(TILEMIX_EINVAL, "too many tokens for one launch");
  p.units = (int32_t)units;
  const dim3 grid((unsigned)((units + kDies - 1) / kDies * kDies));
  if (residual)
    hipLaunchKernelGGL(proj_kernel<true>, grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL(proj_kernel<false>, grid, dim3(kThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TILEMIX_OK : hip_fail(e, residual ? "output projection launch" : "qkv projection launch");
}

int64_t align256(int64_t n) { return (n + 255) & ~int64_t(255); }

// Workspace of one layer: the normalised input (reused for the attention
// output once the projection has read it), Q, K, V, their int8 codes and
// scales, each at a 256-byte boundary.
struct LayerWs {
  int64_t uo, q, k, v, ki, ks, total;
};

LayerWs layer_ws(const int32_t* plan_h) {
  const int64_t T = plan_h[kTotalTokens], hq = plan_h[kHq], hkv = plan_h[kHkv], d = plan_h[kHeadDim];
  LayerWs w;
  int64_t off = 0;
  w.uo = off;
  off += align256(T * hq * d * 2);
  w.q = off;
  off += align256(T * hq * d * 2);
  w.k = off;
  off += align256(T * hkv * d * 2);
  w.v = off;
  off += align256(T * hkv * d * 2);
  w.ki = off;
  off += align256(T * hkv * d);
  w.ks = off;
  off += align256(hkv * (int64_t)plan_h[kTotalKTiles] * 4);
  w.total = off;
  return w;
}

}  // namespace
}  // namespace stack
}  // namespace tilemix

using namespace tilemix;
using namespace tilemix::stack;

extern "C" {

int tilemix_stack_rms_norm(const float* x, void* u_f16, int64_t tokens, int32_t hq, int32_t hkv,
                           int32_t head_dim, float eps, void* hip_stream) {
  clear_error();
  int rc = check_shape(tokens, hq, hkv, head_dim);
  if (rc) return rc;
  if (!(eps >= 0.f)) return fail(TILEMIX_EINVAL, "eps must be >= 0");
  if ((rc = check_ptr(x, "x", tokens > 0)) || (rc = check_ptr(u_f16, "u_f16", tokens > 0))) return rc;
  if (tokens == 0) return TILEMIX_OK;
  return launch_norm(x, static_cast<_Float16*>(u_f16), tokens, hq, hkv, head_dim, eps,
                     static_cast<hipStream_t>(hip_stream));
}

int tilemix_stack_qkv(const void* u_f16, const void* wqkv_f16, void* q_f16, void* k_f16, void* v_f16,
                      int64_t tokens, int32_t hq, int32_t hkv, int32_t head_dim, void* hip_stream) {
  clear_error();
  int rc = check_shape(tokens, hq, hkv, head_dim);
  if (rc) return rc;
  const bool any = tokens > 0;
  if ((rc = check_ptr(u_f16, "u_f16", any)) || (rc = check_ptr(wqkv_f16, "wqkv_f16", any)) ||
      (rc = check_ptr(q_f16, "q_f16", any)) || (rc = check_ptr(k_f16, "k_f16", any)) ||
      (rc = check_ptr(v_f16, "v_f16", any)))
    return rc;
  if (!any) return TILEMIX_OK;
  return launch_proj(false, static_cast<const _Float16*>(u_f16), static_cast<const _Float16*>(wqkv_f16),
                     static_cast<_Float16*>(q_f16), static_cast<_Float16*>(k_f16), static_cast<_Float16*>(v_f16),
                     nullptr, tokens, hq, hkv, head_dim, static_cast<hipStream_t>(hip_stream));
}

int tilemix_stack_out_residual(const void* o_f16, const void* wo_f16, float* x, int64_t tokens, int32_t hq,
                               int32_t hkv, int32_t head_dim, void* hip_stream) {
  clear_error();
  int rc = check_shape(tokens, hq, hkv, head_dim);
  if (rc) return rc;
  const bool any = tokens > 0;
  if ((rc = check_ptr(o_f16, "o_f16", any)) || (rc = check_ptr(wo_f16, "wo_f16", any)) ||
      (rc = check_ptr(x, "x", any)))
    return rc;
  if (!any) return TILEMIX_OK;
  return launch_proj(true, static_cast<const _Float16*>(o_f16), static_cast<const _Float16*>(wo_f16), nullptr,
                     nullptr, nullptr, x, tokens, hq, hkv, head_dim, static_cast<hipStream_t>(hip_stream));
}

int tilemix_stack_workspace_size(const int32_t* plan_h, int64_t* bytes) {
  clear_error();
  int rc = check_plan(plan_h);
  if (rc) return rc;
  if (bytes == nullptr) return fail(TILEMIX_EINVAL, "bytes is NULL");
  *bytes = layer_ws(plan_h).total;
  return TILEMIX_OK;
}

int tilemix_stack_layer(const int32_t* plan_h, const int32_t* plan_d, const uint64_t* words_d, float* x,
                        const void* wqkv_f16, const void* wo_f16, float eps, void* workspace,
                        int64_t workspace_bytes, void* hip_stream) {
  clear_error();
  int rc = check_plans(plan_h, plan_d);
  if (rc) return rc;
  const int64_t T = plan_h[kTotalTokens];
  const int32_t hq = plan_h[kHq], hkv = plan_h[kHkv], d = plan_h[kHeadDim];
  if ((rc = check_shape(T, hq, hkv, d))) return rc;
  if (!(eps >= 0.f)) return fail(TILEMIX_EINVAL, "eps must be >= 0");
  const bool any = T > 0;
  if ((rc = check_ptr(plan_d, "plan_d", true)) || (rc = check_ptr(words_d, "words_d", any)) ||
      (rc = check_ptr(x, "x", any)) || (rc = check_ptr(wqkv_f16, "wqkv_f16", any)) ||
      (rc = check_ptr(wo_f16, "wo_f16", any)) || (rc = check_ptr(workspace, "workspace", any)))
    return rc;
  const LayerWs w = layer_ws(plan_h);
  if (workspace_bytes < w.total)
    return fail(TILEMIX_EINVAL, "workspace holds %lld bytes, needs %lld", (long long)workspace_bytes,
                (long long)w.total);
  if (!any) return TILEMIX_OK;
  char* ws = static_cast<char*>(workspace);
  _Float16* uo = reinterpret_cast<_Float16*>(ws + w.uo);
  _Float16* q = reinterpret_cast<_Float16*>(ws + w.q);
  _Float16* k = reinterpret_cast<_Float16*>(ws + w.k);
  _Float16* v = reinterpret_cast<_Float16*>(ws + w.v);
  int8_t* ki = reinterpret_cast<int8_t*>(ws + w.ki);
  float* ks = reinterpret_cast<float*>(ws + w.ks);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if ((rc = launch_norm(x, uo, T, hq, hkv, d, eps, st))) return rc;
  if ((rc = launch_proj(false, uo, static_cast<const _Float16*>(wqkv_f16), q, k, v, nullptr, T, hq, hkv, d, st)))
    return rc;
  if ((rc = tilemix_quantize_k(plan_h, plan_d, k, ki, ks, hip_stream))) return rc;
  if ((rc = tilemix_prefill_varlen_qinline(plan_h, plan_d, q, k, v, ki, ks, words_d, uo, hip_stream))) return rc;
  return launch_proj(true, uo, static_cast<const _Float16*>(wo_f16), nullptr, nullptr, nullptr, x, T, hq, hkv, d,
                     st);
}

}  // extern "C"
