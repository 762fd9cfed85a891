// Device half of libtilemix for gfx950 (CDNA4): the blockwise Q/K quantiser,
// the fused mixed-precision causal prefill kernel and its int32 tile hook.
//
// Sources (web pages about TileMix), cited by title and section:
//   [Digest]    "TileMix: Tile-Centric Mixed-Precision Attention for LLM
//               Inference Acceleration" (paper digest), method paragraph.
//   [Explainer] "TileMix：给AI大模型的“注意力”做一次精准的精度分配手术"
//               (popular explainer), sections 第二步 and 第三步.
//   [Map]       "Precision Has a Map: TileMix Routes INT8 Inside Dense
//               Attention", section "The routing mechanism is designed to stay
//               inside the hot loop".
//
// Register layouts of the gfx950 matrix instructions used here (lane l of a
// 64-wide wave, c = l % 32, hh = l / 32):
//   v_mfma_f32_32x32x16_f16: A[c][hh*8 + j], B[hh*8 + j][c], j = 0..7
//   v_mfma_i32_32x32x32_i8 : A[c][hh*16 + j], B[hh*16 + j][c], j = 0..15
//   accumulator element i (0..15): C[(i/4)*8 + hh*4 + i%4][c]
// The score tile is computed transposed, S^T = K . Q^T, so that every lane
// owns one query (column c) and the row softmax reduces inside a lane plus
// one exchange with lane l ^ 32.

#include <hip/hip_runtime.h>

#include <cmath>

#include "tilemix.h"
#include "tilemix_host.h"
#include "tilemix_internal.h"

namespace tilemix {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int16v __attribute__((ext_vector_type(16)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int kThreads = 256;  // 4 waves of 64
constexpr float kLog2e = 1.44269504088896340736f;

// --------------------------------------------------------------------------
// Blockwise symmetric quantiser.  [Digest, method]: Q blocks of 128 x d, K
// blocks of 64 x d, scale = absmax / 127, symmetric int8.
// One workgroup per (block, head); the block's values stay in registers
// between the absmax reduction and the rounding pass.
// --------------------------------------------------------------------------
struct QuantArgs {
  const int32_t* plan;
  const _Float16* q;
  const _Float16* k;
  int8_t* qi8;
  int8_t* ki8;
  float* qs;
  float* ks;
  int32_t hq, hkv, batch, tq, tk;
};

__device__ inline int find_seq(const int32_t* seqtab, int batch, int field, int tile) {
  // last sequence whose first tile index is <= tile
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seqtab[mid * kSeqStride + field] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int D, int BLK>
__device__ inline void quantize_block(const _Float16* src, int8_t* dst, float* scale_out,
                                      int row_stride, int nrows, float* red) {
  constexpr int kChunksPerRow = D / 8;                 // 16-byte chunks
  constexpr int kChunks = BLK * kChunksPerRow;
  constexpr int kPerThread = kChunks / kThreads;
  const int tid = threadIdx.x;
  half8 vals[kPerThread];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int idx = tid + i * kThreads;
    const int r = idx / kChunksPerRow, cc = idx % kChunksPerRow;
    half8 v = {};
    if (r < nrows) v = *reinterpret_cast<const half8*>(src + (size_t)r * row_stride + cc * 8);
    vals[i] = v;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((float)v[j]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = __fdiv_rn(amax, 127.0f);
  if (tid == 0) *scale_out = s;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int idx = tid + i * kThreads;
    const int r = idx / kChunksPerRow, cc = idx % kChunksPerRow;
    if (r >= nrows) continue;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int qv = 0;
      if (amax > 0.f) {
        const float qf = __builtin_rintf(__fdiv_rn((float)vals[i][j], s));
        qv = (int)fminf(fmaxf(qf, -127.f), 127.f);
      }
      const uint32_t b = (uint32_t)(qv & 0xff);
      if (j < 4) lo |= b << (8 * j); else hi |= b << (8 * (j - 4));
    }
    *reinterpret_cast<uint2*>(dst + (size_t)r * row_stride + cc * 8) = make_uint2(lo, hi);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void quantize_qk_kernel(QuantArgs a) {
  __shared__ float red[4];
  const int32_t* seqtab = a.plan + kHeaderLen;
  int bid = blockIdx.x;
  const int nq = a.tq * a.hq;
  if (bid < nq) {
    const int tile = bid / a.hq, head = bid % a.hq;
    const int s = find_seq(seqtab, a.batch, kSeqQtOff, tile);
    const int32_t* rec = seqtab + s * kSeqStride;
    const int local = tile - rec[kSeqQtOff];
    const int row0 = rec[kSeqStart] + local * kBlockM;
    const int nrows = min(kBlockM, rec[kSeqLen] - local * kBlockM);
    const size_t base = ((size_t)row0 * a.hq + head) * D;
    quantize_block<D, kBlockM>(a.q + base, a.qi8 + base, a.qs + (size_t)head * a.tq + tile,
                               a.hq * D, nrows, red);
  } else {
    bid -= nq;
    const int tile = bid / a.hkv, head = bid % a.hkv;
    const int s = find_seq(seqtab, a.batch, kSeqKtOff, tile);
    const int32_t* rec = seqtab + s * kSeqStride;
    const int local = tile - rec[kSeqKtOff];
    const int row0 = rec[kSeqStart] + local * kBlockN;
    const int nrows = min(kBlockN, rec[kSeqLen] - local * kBlockN);
    const size_t base = ((size_t)row0 * a.hkv + head) * D;
    quantize_block<D, kBlockN>(a.k + base, a.ki8 + base, a.ks + (size_t)head * a.tk + tile,
                               a.hkv * D, nrows, red);
  }
}

// --------------------------------------------------------------------------
// Fused prefill pieces shared by the kernel and the int32 tile hook.
// --------------------------------------------------------------------------
template <int D>
struct Lds {
  static constexpr int kKStride = D + 8;     // halfs per fp16 K row (pads 16 B)
  static constexpr int kK8Stride = D + 16;   // bytes per int8 K row (pads 16 B)
  static constexpr int kVStride = D + 16;    // halfs per V row (pads 32 B)
  static constexpr int kKBytes = kBlockN * kKStride * 2;
  static constexpr int kVBytes = kBlockN * kVStride * 2;
};

// Stage one 64-key tile of int8 K into LDS; rows past the sequence end are 0.
template <int D>
__device__ inline void stage_k_i8(char* sK, const int8_t* k_rows, int row_stride, int nvalid) {
  constexpr int kChunksPerRow = D / 16;
  constexpr int kChunks = kBlockN * kChunksPerRow;
  for (int idx = threadIdx.x; idx < kChunks; idx += kThreads) {
    const int r = idx / kChunksPerRow, cc = idx % kChunksPerRow;
    int4v v = {0, 0, 0, 0};
    if (r < nvalid) v = *reinterpret_cast<const int4v*>(k_rows + (size_t)r * row_stride + cc * 16);
    *reinterpret_cast<int4v*>(sK + r * Lds<D>::kK8Stride + cc * 16) = v;
  }
}

// Stage one 64-row fp16 tile (K or V) into LDS with the given row stride.
template <int D, int kStride>
__device__ inline void stage_f16(_Float16* sX, const _Float16* rows, int row_stride, int nvalid) {
  constexpr int kChunksPerRow = D / 8;
  constexpr int kChunks = kBlockN * kChunksPerRow;
  for (int idx = threadIdx.x; idx < kChunks; idx += kThreads) {
    const int r = idx / kChunksPerRow, cc = idx % kChunksPerRow;
    half8 v = {};
    if (r < nvalid) v = *reinterpret_cast<const half8*>(rows + (size_t)r * row_stride + cc * 8);
    *reinterpret_cast<half8*>(sX + r * kStride + cc * 8) = v;
  }
}

// INT8 path of one wave's 64 x 32 score block: S^T = K_i8 . Q_i8^T with int32
// accumulation ([Digest, method]: INT8 MMA, INT32 accumulation).
template <int D>
__device__ inline void qk_tile_i8(const char* sK, const int4v* qb, int16v acc[2]) {
  const int lane = threadIdx.x & 63, c = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    int16v a = {};
    const char* row = sK + (kb * 32 + c) * Lds<D>::kK8Stride + hh * 16;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const int4v kf = *reinterpret_cast<const int4v*>(row + kk * 32);
      a = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qb[kk], a, 0, 0, 0);
    }
    acc[kb] = a;
  }
}

// FP16 path of the same block: S^T = K . Q^T, fp32 accumulation.
template <int D>
__device__ inline void qk_tile_f16(const _Float16* sK, const half8* qf, float16v acc[2]) {
  const int lane = threadIdx.x & 63, c = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    float16v a = {};
    const _Float16* row = sK + (kb * 32 + c) * Lds<D>::kKStride + hh * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const half8 kf = *reinterpret_cast<const half8*>(row + kk * 16);
      a = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[kk], a, 0, 0, 0);
    }
    acc[kb] = a;
  }
}

// Query fragments of this lane's query row (zeros outside the sequence).
template <int D>
__device__ inline void load_q(const _Float16* qrow, const int8_t* q8row, bool valid, half8* qf,
                              int4v* qb) {
  const int hh = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    half8 v = {};
    if (valid) v = *reinterpret_cast<const half8*>(qrow + kk * 16 + hh * 8);
    qf[kk] = v;
  }
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    int4v v = {0, 0, 0, 0};
    if (valid) v = *reinterpret_cast<const int4v*>(q8row + kk * 32 + hh * 16);
    qb[kk] = v;
  }
}

// --------------------------------------------------------------------------
// Fused mixed-precision prefill.  One workgroup = one work unit (sequence,
// query head, 128-row query tile); wave w owns queries 32w .. 32w+31.
// Per legal key tile: routing bit lookup ([Map, hot loop]: shift and mask),
// QK^T on the routed path, rescale into the common score domain ([Explainer,
// 第三步]), causal/sequence-end mask, shared online softmax, P.V in FP16
// ([Digest, method]).
// --------------------------------------------------------------------------
struct PrefillArgs {
  const int32_t* plan;
  const _Float16* q;
  const _Float16* k;
  const _Float16* v;
  const int8_t* qi8;
  const int8_t* ki8;
  const float* qs;
  const float* ks;
  const uint64_t* words;
  _Float16* out;
  int32_t hq, hkv, tq, tk;
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char sK[Lds<D>::kKBytes];
  __shared__ __attribute__((aligned(16))) _Float16 sV[kBlockN * Lds<D>::kVStride];

  const int32_t* item = a.plan + a.plan[kItemOff] + kItemStride * blockIdx.x;
  const int seq = item[0];
  if (seq < 0) return;
  const int head = item[1] >> 16, row = item[1] & 0xffff;
  const int32_t* rec = a.plan + kHeaderLen + seq * kSeqStride;
  const int start = rec[kSeqStart], L = rec[kSeqLen], qt_off = rec[kSeqQtOff];
  const int kt_off = rec[kSeqKtOff], g = rec[kSeqG];
  const int kv = head / (a.hq / a.hkv);
  const int q0 = row * kBlockM;
  const int last_tile = min(q0 + kBlockM - 1, L - 1) / kBlockN;
  const uint64_t word = a.words[(size_t)kv * a.tq + qt_off + row];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, c = lane & 31, hh = lane >> 5;
  const int qi = q0 + 32 * w + c;  // this lane's query (sequence-local)
  const bool qvalid = qi < L;

  half8 qf[D / 16];
  int4v qb[D / 32];
  load_q<D>(a.q + ((size_t)(start + qi) * a.hq + head) * D,
            a.qi8 + ((size_t)(start + qi) * a.hq + head) * D, qvalid, qf, qb);
  const float sq = a.qs[(size_t)head * a.tq + qt_off + row];
  const float inv_sqrt_d = (float)(1.0 / std::sqrt((double)D));
  const float scale16 = inv_sqrt_d * kLog2e;

  float m = -INFINITY, lsum = 0.f;
  float16v o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = (float16v){};

  const int kv_stride = a.hkv * D;
  for (int t = 0; t <= last_tile; ++t) {
    const int bit = (int)((word >> (t / g)) & 1ull);
    const int k0 = t * kBlockN;
    const int nvalid = min(kBlockN, L - k0);
    const size_t krow = ((size_t)(start + k0) * a.hkv + kv) * D;
    __syncthreads();  // previous tile's LDS reads are done
    if (bit) stage_k_i8<D>(sK, a.ki8 + krow, kv_stride, nvalid);
    else stage_f16<D, Lds<D>::kKStride>(reinterpret_cast<_Float16*>(sK), a.k + krow, kv_stride, nvalid);
    stage_f16<D, Lds<D>::kVStride>(sV, a.v + krow, kv_stride, nvalid);
    __syncthreads();

    // Scores of this wave's 32 queries x 64 keys, in the log2 domain.
    float x[2][16];
    if (bit) {
      int16v acc[2];
      qk_tile_i8<D>(sK, qb, acc);
      const float sk = a.ks[(size_t)kv * a.tk + kt_off + t];
      const float f = (sq * sk) * inv_sqrt_d * kLog2e;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) x[kb][i] = (float)acc[kb][i] * f;
    } else {
      float16v acc[2];
      qk_tile_f16<D>(reinterpret_cast<const _Float16*>(sK), qf, acc);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) x[kb][i] = acc[kb][i] * scale16;
    }
    // Causal / sequence-end mask, independent of the routing bit.
    if (k0 + kBlockN - 1 > q0 || k0 + kBlockN > L) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
          if (key > qi || key >= L) x[kb][i] = -INFINITY;
        }
    }
    // Shared online softmax state.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, x[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    half8 p[2][2];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const half2v pk = {(_Float16)__builtin_amdgcn_exp2f(x[kb][i] - m_new),
                           (_Float16)__builtin_amdgcn_exp2f(x[kb][i + 1] - m_new)};
        psum = __builtin_amdgcn_fdot2(pk, (half2v){(_Float16)1.0f, (_Float16)1.0f}, psum, false);
        p[kb][i >> 3][i & 7] = pk[0];
        p[kb][i >> 3][(i & 7) + 1] = pk[1];
      }
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;

    // O^T += V^T . P^T (fp16 operands, fp32 accumulation).
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kbase = ks * 16;
      const int j = lane & 15, sub = (lane >> 4) & 1;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const _Float16* p0 = sV + (kbase + hh * 4 + (j >> 2)) * Lds<D>::kVStride + db * 32 + sub * 16 + 4 * (j & 3);
        // Whole-vector casts: element-wise extraction of the transposed
        // read's result is mis-assembled by this compiler.
        const half4 lo = __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(short4v, p0)));
        const half4 hi = __builtin_bit_cast(
            half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(short4v, p0 + 8 * Lds<D>::kVStride)));
        const half8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, p[ks >> 1][ks & 1], o[db], 0, 0, 0);
      }
    }
  }

  // Epilogue: O = acc / l, fp16 round-to-nearest-even.
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = 1.0f / ltot;
  if (qvalid) {
    _Float16* orow = a.out + ((size_t)(start + qi) * a.hq + head) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        half4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = (_Float16)(o[db][i4 * 4 + e] * inv);
        *reinterpret_cast<half4*>(orow + db * 32 + i4 * 8 + hh * 4) = h;
      }
  }
}

// Int32 accumulator of one INT8 score tile, through the kernel's own
// staging and qk_tile_i8 routine.
template <int D>
__global__ __launch_bounds__(kThreads) void debug_qk_i32_kernel(const int32_t* plan, const int8_t* qi8,
                                                                const int8_t* ki8, int seq, int head,
                                                                int row, int t, int32_t* acc_out) {
  __shared__ __attribute__((aligned(16))) char sK[Lds<D>::kKBytes];
  const int hq = plan[kHq], hkv = plan[kHkv];
  const int32_t* rec = plan + kHeaderLen + seq * kSeqStride;
  const int start = rec[kSeqStart], L = rec[kSeqLen];
  const int kv = head / (hq / hkv);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, c = lane & 31, hh = lane >> 5;
  const int qi = row * kBlockM + 32 * w + c;
  const int k0 = t * kBlockN;
  stage_k_i8<D>(sK, ki8 + ((size_t)(start + k0) * hkv + kv) * D, hkv * D, max(0, min(kBlockN, L - k0)));
  int4v qb[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    int4v v = {0, 0, 0, 0};
    if (qi < L)
      v = *reinterpret_cast<const int4v*>(qi8 + ((size_t)(start + qi) * hq + head) * D + kk * 32 + hh * 16);
    qb[kk] = v;
  }
  __syncthreads();
  int16v acc[2];
  qk_tile_i8<D>(sK, qb, acc);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kb * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
      acc_out[(32 * w + c) * kBlockN + key] = acc[kb][i];
    }
}

}  // namespace tilemix

using namespace tilemix;

namespace {

int hip_fail(hipError_t e, const char* what) {
  return fail(TILEMIX_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int check_dev_ptr(const void* p, const char* name, bool needed) {
  if (!needed) return TILEMIX_OK;
  if (p == nullptr) return fail(TILEMIX_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(TILEMIX_EINVAL, "%s is not 16-byte aligned", name);
  return TILEMIX_OK;
}

}  // namespace

extern "C" {

int tilemix_quantize_qk(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                        const void* k_f16, int8_t* q_i8, int8_t* k_i8, float* q_scale,
                        float* k_scale, void* hip_stream) {
  clear_error();
  int rc = check_plan(plan_h);
  if (rc) return rc;
  const bool any = plan_h[kTotalTokens] > 0;
  if ((rc = check_dev_ptr(plan_d, "plan_d", true)) || (rc = check_dev_ptr(q_f16, "q_f16", any)) ||
      (rc = check_dev_ptr(k_f16, "k_f16", any)) || (rc = check_dev_ptr(q_i8, "q_i8", any)) ||
      (rc = check_dev_ptr(k_i8, "k_i8", any)) || (rc = check_dev_ptr(q_scale, "q_scale", any)) ||
      (rc = check_dev_ptr(k_scale, "k_scale", any)))
    return rc;
  if (!any) return TILEMIX_OK;
  QuantArgs a;
  a.plan = plan_d;
  a.q = static_cast<const _Float16*>(q_f16);
  a.k = static_cast<const _Float16*>(k_f16);
  a.qi8 = q_i8;
  a.ki8 = k_i8;
  a.qs = q_scale;
  a.ks = k_scale;
  a.hq = plan_h[kHq];
  a.hkv = plan_h[kHkv];
  a.batch = plan_h[kBatch];
  a.tq = plan_h[kTotalQTiles];
  a.tk = plan_h[kTotalKTiles];
  const int64_t blocks = (int64_t)a.tq * a.hq + (int64_t)a.tk * a.hkv;
  if (blocks > 0x7fffffff) return fail(TILEMIX_EINVAL, "batch too large for one launch");
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (plan_h[kHeadDim] == 64)
    hipLaunchKernelGGL(quantize_qk_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(quantize_qk_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  return TILEMIX_OK;
}

int tilemix_prefill_varlen(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                           const void* k_f16, const void* v_f16, const int8_t* q_i8,
                           const int8_t* k_i8, const float* q_scale, const float* k_scale,
                           const uint64_t* words_d, void* out_f16, void* hip_stream) {
  clear_error();
  int rc = check_plan(plan_h);
  if (rc) return rc;
  const bool any = plan_h[kNumItems] > 0;
  if ((rc = check_dev_ptr(plan_d, "plan_d", true)) || (rc = check_dev_ptr(q_f16, "q_f16", any)) ||
      (rc = check_dev_ptr(k_f16, "k_f16", any)) || (rc = check_dev_ptr(v_f16, "v_f16", any)) ||
      (rc = check_dev_ptr(q_i8, "q_i8", any)) || (rc = check_dev_ptr(k_i8, "k_i8", any)) ||
      (rc = check_dev_ptr(q_scale, "q_scale", any)) || (rc = check_dev_ptr(k_scale, "k_scale", any)) ||
      (rc = check_dev_ptr(words_d, "words_d", any)) || (rc = check_dev_ptr(out_f16, "out_f16", any)))
    return rc;
  if (!any) return TILEMIX_OK;
  PrefillArgs a;
  a.plan = plan_d;
  a.q = static_cast<const _Float16*>(q_f16);
  a.k = static_cast<const _Float16*>(k_f16);
  a.v = static_cast<const _Float16*>(v_f16);
  a.qi8 = q_i8;
  a.ki8 = k_i8;
  a.qs = q_scale;
  a.ks = k_scale;
  a.words = words_d;
  a.out = static_cast<_Float16*>(out_f16);
  a.hq = plan_h[kHq];
  a.hkv = plan_h[kHkv];
  a.tq = plan_h[kTotalQTiles];
  a.tk = plan_h[kTotalKTiles];
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const unsigned grid = (unsigned)plan_h[kNumItems];
  if (plan_h[kHeadDim] == 64)
    hipLaunchKernelGGL(prefill_kernel<64>, dim3(grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(prefill_kernel<128>, dim3(grid), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return TILEMIX_OK;
}

int tilemix_debug_qk_i32_tile(const int32_t* plan_h, const int32_t* plan_d, const int8_t* q_i8,
                              const int8_t* k_i8, int32_t seq, int32_t head, int32_t r, int32_t t,
                              int32_t* acc_d, void* hip_stream) {
  clear_error();
  int rc = check_plan(plan_h);
  if (rc) return rc;
  if ((rc = check_dev_ptr(plan_d, "plan_d", true)) || (rc = check_dev_ptr(q_i8, "q_i8", true)) ||
      (rc = check_dev_ptr(k_i8, "k_i8", true)) || (rc = check_dev_ptr(acc_d, "acc_d", true)))
    return rc;
  if (seq < 0 || seq >= plan_h[kBatch]) return fail(TILEMIX_EINVAL, "seq %d out of range", seq);
  if (head < 0 || head >= plan_h[kHq]) return fail(TILEMIX_EINVAL, "head %d out of range", head);
  const int32_t* rec = plan_h + kHeaderLen + seq * kSeqStride;
  if (r < 0 || r >= rec[kSeqTm]) return fail(TILEMIX_EINVAL, "row %d out of range", r);
  if (t < 0 || t >= rec[kSeqTn]) return fail(TILEMIX_EINVAL, "key tile %d out of range", t);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (plan_h[kHeadDim] == 64)
    hipLaunchKernelGGL(debug_qk_i32_kernel<64>, dim3(1), dim3(kThreads), 0, st, plan_d, q_i8, k_i8,
                       seq, head, r, t, acc_d);
  else
    hipLaunchKernelGGL(debug_qk_i32_kernel<128>, dim3(1), dim3(kThreads), 0, st, plan_d, q_i8, k_i8,
                       seq, head, r, t, acc_d);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "debug tile launch");
  return TILEMIX_OK;
}

}  // extern "C"
