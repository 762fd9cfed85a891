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

#include <cfloat>
#include <cmath>
#include <type_traits>

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
typedef int int8v __attribute__((ext_vector_type(8)));

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

// q = round-half-even(fl32(x / s)) clamped to [-127, 127].  x * fl32(1 / s)
// is within 2.3e-5 of fl32(x / s) for |x / s| <= 127 (two roundings of 2^-24
// relative each plus half an ulp of the quotient), so it rounds to the same
// integer unless it lies within 2^-15 of a half-integer; only those elements
// take the exact IEEE division.  rs = fl32(1 / s), or 0 when s = 0.
__device__ inline int quant_code_i8(float x, float rs, float s) {
  const float y = x * rs;
  float qf = __builtin_rintf(y);
  if (__builtin_fabsf(y - qf) > 0.5f - 0x1p-15f) qf = __builtin_rintf(__fdiv_rn(x, s));
  return (int)__builtin_amdgcn_fmed3f(qf, -127.f, 127.f);
}

// The block's absmax over the values this thread holds (thread tid holds
// the 16-byte chunks tid + i * kThreads of the block, rows past the block's
// end as zeros), its scale, and the codes of the rows before the end.
template <int D, int BLK>
__device__ inline void quantize_store(const half8 (&vals)[BLK * (D / 8) / kThreads], int8_t* dst, float* scale_out,
                                      int row_stride, int nrows, float* red) {
  constexpr int kChunksPerRow = D / 8;                 // 16-byte chunks
  constexpr int kPerThread = BLK * kChunksPerRow / kThreads;
  const int tid = threadIdx.x;
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((float)vals[i][j]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = __fdiv_rn(amax, 127.0f);
  if (tid == 0) *scale_out = s;
  const float rs = amax > 0.f ? __fdiv_rn(1.0f, s) : 0.f;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int idx = tid + i * kThreads;
    const int r = idx / kChunksPerRow, cc = idx % kChunksPerRow;
    if (r >= nrows) continue;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t b = (uint32_t)(quant_code_i8((float)vals[i][j], rs, s) & 0xff);
      if (j < 4) lo |= b << (8 * j); else hi |= b << (8 * (j - 4));
    }
    *reinterpret_cast<uint2*>(dst + (size_t)r * row_stride + cc * 8) = make_uint2(lo, hi);
  }
}

template <int D, int BLK>
__device__ inline void quantize_block(const _Float16* src, int8_t* dst, float* scale_out,
                                      int row_stride, int nrows, float* red) {
  constexpr int kChunksPerRow = D / 8;                 // 16-byte chunks
  constexpr int kPerThread = BLK * kChunksPerRow / kThreads;
  const int tid = threadIdx.x;
  half8 vals[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int idx = tid + i * kThreads;
    const int r = idx / kChunksPerRow, cc = idx % kChunksPerRow;
    half8 v = {};
    if (r < nrows) v = *reinterpret_cast<const half8*>(src + (size_t)r * row_stride + cc * 8);
    vals[i] = v;
  }
  quantize_store<D, BLK>(vals, dst, scale_out, row_stride, nrows, red);
}

// Key blocks alone, one workgroup per (key tile of a sequence, KV head) with
// the sequence taken from the grid (no search over the sequence table) and
// the KV head fastest in the launch order (neighbouring workgroups read
// neighbouring bytes of the same rows).  The block's rows come through a
// buffer resource sized to the rows before the sequence end, so every load
// is issued at once without a branch (rows past the end read as zero, as
// quantize_block's guarded loads give them).  Codes and scales are those of
// quantize_block, bit for bit.
template <int D>
__global__ __launch_bounds__(kThreads) void quantize_k_kernel(QuantArgs a) {
  __shared__ float red[4];
  constexpr int kChunksPerRow = D / 8;
  constexpr int kPerThread = kBlockN * kChunksPerRow / kThreads;
  const int head = blockIdx.x % a.hkv, local = blockIdx.x / a.hkv, seq = blockIdx.y;
  const int32_t* rec = a.plan + kHeaderLen + seq * kSeqStride;
  const int L = rec[kSeqLen];
  if (local * kBlockN >= L) return;
  const int nrows = min(kBlockN, L - local * kBlockN);
  const int stride = a.hkv * D;  // elements between consecutive rows
  const size_t base = ((size_t)(rec[kSeqStart] + local * kBlockN) * a.hkv + head) * D;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.k + base), (short)0, (int)((size_t)nrows * stride * sizeof(_Float16)), 0x00020000);
  half8 vals[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int idx = threadIdx.x + i * kThreads;
    const int r = idx / kChunksPerRow, cc = idx % kChunksPerRow;
    vals[i] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(
                                            rs, (uint32_t)((r * stride + cc * 8) * sizeof(_Float16)), 0, 0));
  }
  quantize_store<D, kBlockN>(vals, a.ki8 + base, a.ks + (size_t)head * a.tk + rec[kSeqKtOff] + local, stride,
                             nrows, red);
}

template <int D>
__global__ __launch_bounds__(kThreads) void quantize_qk_kernel(QuantArgs a) {
  __shared__ float red[4];
  const int32_t* seqtab = a.plan + kHeaderLen;
  int bid = blockIdx.x;
  const int nq = a.q ? a.tq * a.hq : 0;  // no Q pointer: the key blocks only
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
// FP8 (E4M3) blockwise quantiser: the same blocks, s = fl32(absmax / 448),
// code = E4M3 round-half-even of fl32(x / s) (the hardware conversion rounds
// to nearest even and |x / s| <= 448); an all-zero block has s = 0 and codes
// 0.
// --------------------------------------------------------------------------
template <int D, int BLK>
__device__ inline void quantize_block_fp8(const _Float16* src, uint8_t* dst, float* scale_out, int row_stride,
                                          int nrows, float* red) {
  constexpr int kChunksPerRow = D / 8;
  constexpr int kPerThread = BLK * kChunksPerRow / kThreads;
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
  const float s = __fdiv_rn(amax, 448.0f);
  if (tid == 0) *scale_out = s;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int idx = tid + i * kThreads;
    const int r = idx / kChunksPerRow, cc = idx % kChunksPerRow;
    if (r >= nrows) continue;
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = amax > 0.f ? __fdiv_rn((float)vals[i][j], s) : 0.f;
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
    *reinterpret_cast<uint2*>(dst + (size_t)r * row_stride + cc * 8) = make_uint2((uint32_t)lo, (uint32_t)hi);
  }
}

// Both key codes of one block from a single read: the INT8 codes of
// quantize_block and the E4M3 codes of quantize_block_fp8, element for
// element the same arithmetic, from the one absmax.
template <int D, int BLK>
__device__ inline void quantize_block_i8_fp8(const _Float16* src, int8_t* dst8, uint8_t* dstf, float* scale8,
                                             float* scalef, int row_stride, int nrows, float* red) {
  constexpr int kChunksPerRow = D / 8;
  constexpr int kPerThread = BLK * kChunksPerRow / kThreads;
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
  const float s8 = __fdiv_rn(amax, 127.0f);
  const float sf = __fdiv_rn(amax, 448.0f);
  if (tid == 0) {
    *scale8 = s8;
    *scalef = sf;
  }
  const float rs8 = amax > 0.f ? __fdiv_rn(1.0f, s8) : 0.f;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int idx = tid + i * kThreads;
    const int r = idx / kChunksPerRow, cc = idx % kChunksPerRow;
    if (r >= nrows) continue;
    uint32_t lo = 0, hi = 0;
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t b = (uint32_t)(quant_code_i8((float)vals[i][j], rs8, s8) & 0xff);
      if (j < 4) lo |= b << (8 * j); else hi |= b << (8 * (j - 4));
      y[j] = amax > 0.f ? __fdiv_rn((float)vals[i][j], sf) : 0.f;
    }
    *reinterpret_cast<uint2*>(dst8 + (size_t)r * row_stride + cc * 8) = make_uint2(lo, hi);
    int flo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    flo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], flo, true);
    int fhi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    fhi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], fhi, true);
    *reinterpret_cast<uint2*>(dstf + (size_t)r * row_stride + cc * 8) = make_uint2((uint32_t)flo, (uint32_t)fhi);
  }
}

struct QuantKBothArgs {
  const int32_t* plan;
  const _Float16* k;
  int8_t* ki8;
  uint8_t* kf8;
  float* ks;
  float* ksf8;
  int32_t hkv, batch, tk;
};

// One workgroup per (key block, KV head).
template <int D>
__global__ __launch_bounds__(kThreads) void quantize_k_i8_fp8_kernel(QuantKBothArgs a) {
  __shared__ float red[4];
  const int32_t* seqtab = a.plan + kHeaderLen;
  const int bid = blockIdx.x;
  const int tile = bid / a.hkv, head = bid % a.hkv;
  const int s = find_seq(seqtab, a.batch, kSeqKtOff, tile);
  const int32_t* rec = seqtab + s * kSeqStride;
  const int local = tile - rec[kSeqKtOff];
  const int row0 = rec[kSeqStart] + local * kBlockN;
  const int nrows = min(kBlockN, rec[kSeqLen] - local * kBlockN);
  const size_t base = ((size_t)row0 * a.hkv + head) * D;
  quantize_block_i8_fp8<D, kBlockN>(a.k + base, a.ki8 + base, a.kf8 + base, a.ks + (size_t)head * a.tk + tile,
                                    a.ksf8 + (size_t)head * a.tk + tile, a.hkv * D, nrows, red);
}

struct QuantFp8Args {
  const int32_t* plan;
  const _Float16* q;
  const _Float16* k;
  uint8_t* qf8;
  uint8_t* kf8;
  float* qs;
  float* ks;
  int32_t hq, hkv, batch, tq, tk;
};

template <int D>
__global__ __launch_bounds__(kThreads) void quantize_qk_fp8_kernel(QuantFp8Args a) {
  __shared__ float red[4];
  const int32_t* seqtab = a.plan + kHeaderLen;
  int bid = blockIdx.x;
  const int nq = a.q ? a.tq * a.hq : 0;  // no Q pointer: the key blocks only
  if (bid < nq) {
    const int tile = bid / a.hq, head = bid % a.hq;
    const int s = find_seq(seqtab, a.batch, kSeqQtOff, tile);
    const int32_t* rec = seqtab + s * kSeqStride;
    const int local = tile - rec[kSeqQtOff];
    const int row0 = rec[kSeqStart] + local * kBlockM;
    const int nrows = min(kBlockM, rec[kSeqLen] - local * kBlockM);
    const size_t base = ((size_t)row0 * a.hq + head) * D;
    quantize_block_fp8<D, kBlockM>(a.q + base, a.qf8 + base, a.qs + (size_t)head * a.tq + tile, a.hq * D,
                                   nrows, red);
  } else {
    bid -= nq;
    const int tile = bid / a.hkv, head = bid % a.hkv;
    const int s = find_seq(seqtab, a.batch, kSeqKtOff, tile);
    const int32_t* rec = seqtab + s * kSeqStride;
    const int local = tile - rec[kSeqKtOff];
    const int row0 = rec[kSeqStart] + local * kBlockN;
    const int nrows = min(kBlockN, rec[kSeqLen] - local * kBlockN);
    const size_t base = ((size_t)row0 * a.hkv + head) * D;
    quantize_block_fp8<D, kBlockN>(a.k + base, a.kf8 + base, a.ks + (size_t)head * a.tk + tile, a.hkv * D,
                                   nrows, red);
  }
}

// --------------------------------------------------------------------------
// Fused prefill pieces shared by the kernel and the int32 tile hook.
//
// LDS holds two tile buffers (double buffering); a buffer is one K tile
// (fp16, or int8 on INT8-routed tiles) followed by one fp16 V tile, 64 rows
// each.  Tiles arrive by direct buffer->LDS loads (buffer_load_dwordx4 ...
// lds): lane i of a wave writes bytes [16 i, 16 i + 16) of a 1 KiB window.
// A tile of R rows per window uses NW = 64 / R windows; row r lives in
// window r % NW at slot r / NW, and consecutive windows are kWinPad bytes
// further apart than 1 KiB.  Rows r .. r+NW-1 therefore start on shifted
// banks, which makes the fragment reads below conflict-free with purely
// additive addresses (lane part + compile-time offset):
//   K rows (fp16 or int8): window pitch 1040 B -> 16 consecutive rows at one
//     16-byte column start 4 banks apart;
//   V rows: window pitch 1088 B -> the 4 rows x 64 B read by 32 lanes of a
//     transposed read start 16 banks apart.
// --------------------------------------------------------------------------
// Buffer resource for raw (unstrided) byte addressing from `base`.
__device__ inline int4v make_rsrc(const void* base) {
  const unsigned long long b = reinterpret_cast<unsigned long long>(base);
  return (int4v){(int)__builtin_amdgcn_readfirstlane((unsigned)b),
                 (int)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32) & 0xffffu), 0x7fffffff, 0x00020000};
}

// One direct buffer->LDS load: every lane's 16 bytes at (voffset + soffset)
// land at lds_dst + 16 * lane.  Written as inline asm on purpose: the
// compiler's own form makes every later LDS read wait for all such loads in
// flight (it cannot tell the two tile buffers apart), which would serialise
// the prefetch.  Completion is awaited explicitly (wait_tile_loads) before the
// barrier that publishes the tile.
__device__ inline void lds_dma16(char* lds_dst, int4v rsrc, int voffset, int soffset) {
  const unsigned la = __builtin_amdgcn_readfirstlane((unsigned)(size_t)LDS_PTR(char, lds_dst));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(la), "v"(voffset),
               "s"(rsrc), "s"(soffset)
               : "memory", "m0");
}

// The same load into a wave-uniform LDS byte address.
__device__ inline void lds_dma16_at(unsigned lds, int4v rsrc, int voffset, int soffset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voffset),
               "s"(rsrc), "s"(soffset)
               : "memory", "m0");
}

template <int kRowBytes, int kPitch>
struct Layout {
  static constexpr int kRowsPerWin = 1024 / kRowBytes;
  static constexpr int kWins = kBlockN / kRowsPerWin;
  static constexpr int kBytes = kWins * kPitch;
  static constexpr int kLanesPerRow = kRowBytes / 16;
  // LDS byte offset of (row, byte column) within the tile.
  __device__ static constexpr int at(int row, int col) {
    return (row % kWins) * kPitch + (row / kWins) * kRowBytes + col;
  }
  // Lane part of the source offset of this lane's 16 bytes in every window
  // (window j adds j * row stride).
  __device__ static int lane_src(int lane, int gstride) {
    return (lane / kLanesPerRow) * kWins * gstride + (lane % kLanesPerRow) * 16;
  }
  // A tile of 64 rows inside the sequence: this wave's windows (the windows
  // split evenly over the four waves), addressed from the tile's LDS byte
  // address `lds_tile` without per-window checks.
  __device__ static void issue_full(unsigned lds_tile, const void* base, int gstride, int wave, int lane_off) {
    static_assert(kWins % 4 == 0, "windows split evenly over the four waves");
    const int4v rsrc = make_rsrc(base);
#pragma unroll
    for (int i = 0; i < kWins / 4; ++i) {
      const int j = wave + 4 * i;
      lds_dma16_at(lds_tile + j * kPitch, rsrc, lane_off, j * gstride);
    }
  }
  // Issue the tile whose first row is at `base`; rows >= nvalid repeat row
  // nvalid - 1 of the same sequence (finite; those keys are masked).
  __device__ static void issue(char* lds_tile, const void* base, int gstride, int nvalid, int wave,
                               int lane, int lane_off) {
    const int4v rsrc = make_rsrc(base);
    if (nvalid == kBlockN) {
#pragma unroll
      for (int i = 0; i < (kWins + 3) / 4; ++i) {
        const int j = wave + 4 * i;
        if (j < kWins) lds_dma16(lds_tile + j * kPitch, rsrc, lane_off, j * gstride);
      }
    } else {
      // last tile of a sequence: clamp the row
#pragma unroll
      for (int i = 0; i < (kWins + 3) / 4; ++i) {
        const int j = wave + 4 * i;
        if (j < kWins) {
          const int r = min(j + (lane / kLanesPerRow) * kWins, nvalid - 1);
          lds_dma16(lds_tile + j * kPitch, rsrc, r * gstride + (lane % kLanesPerRow) * 16, 0);
        }
      }
    }
  }
};

template <int D>
struct Tile {
  using K16 = Layout<2 * D, 1040>;
  using K8 = Layout<D, 1040>;
  using V = Layout<2 * D, 1088>;
  static constexpr int kKRegion = K16::kBytes > K8::kBytes ? K16::kBytes : K8::kBytes;
  static constexpr int kBuf = kKRegion + V::kBytes;
  static constexpr int kScales = 1024;  // key-tile scales staged per chunk
  static constexpr int kLds = 2 * kBuf + kScales * 4;
  static constexpr int kLds3 = kLds + kScales * 4;  // + the FP8 key-tile scales
  static constexpr int kLdsQ = kLds + 16;             // + the Q absmax exchange
  static constexpr int kLds3Q = kLds3 + 16;
};

// Combine a value with the same register of lane l ^ 32 (no LDS round trip).
__device__ inline float max_with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline void wait_tile_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wave-uniform read-only scalar: read through the constant address space so
// it becomes a scalar load (waited on by lgkmcnt, not vmcnt, so it does not
// wait for the tile loads in flight).
__device__ inline float load_uniform(const float* p) {
  return *(const __attribute__((address_space(4))) float*)(p);
}

// The fragment reads below are issued one batch ahead of the matrix
// instructions that consume them, with scheduling fences so the compiler
// keeps that order (left alone it sinks each read next to its consumer and
// exposes the full LDS latency on every instruction).
#define TM_FENCE() __builtin_amdgcn_sched_barrier(0)

// INT8 path of one wave's 64 x 32 score block: S^T = K_i8 . Q_i8^T with int32
// accumulation ([Digest, method]: INT8 MMA, INT32 accumulation).
template <int D>
__device__ inline void qk_tile_i8(const char* sK, const int4v* qb, int16v acc[2]) {
  using K8 = typename Tile<D>::K8;
  constexpr int kSteps = D / 32;               // per 32-key block
  constexpr int kBatch = kSteps < 4 ? kSteps : 4;
  constexpr int kBatches = 2 * kSteps / kBatch;
  const int lane = threadIdx.x & 63, c = lane & 31, hh = lane >> 5;
  const char* base = sK + K8::at(c, hh * 16);
  int4v kf[2][kBatch];
  auto load = [&](int bt, int4v* dst) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int step = bt * kBatch + i, kb = step / kSteps, kk = step % kSteps;
      dst[i] = *reinterpret_cast<const int4v*>(base + K8::at(kb * 32, kk * 32));
    }
  };
  acc[0] = (int16v){};
  acc[1] = (int16v){};
  load(0, kf[0]);
#pragma unroll
  for (int bt = 0; bt < kBatches; ++bt) {
    TM_FENCE();
    if (bt + 1 < kBatches) load(bt + 1, kf[(bt + 1) & 1]);
    TM_FENCE();
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int step = bt * kBatch + i, kb = step / kSteps, kk = step % kSteps;
      acc[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[bt & 1][i], qb[kk], acc[kb], 0, 0, 0);
    }
  }
  TM_FENCE();
}

// FP16 path of the same block: S^T = K . Q^T, fp32 accumulation.
template <int D>
__device__ inline void qk_tile_f16(const char* sK, const half8* qf, float16v acc[2]) {
  using K16 = typename Tile<D>::K16;
  constexpr int kSteps = D / 16;               // per 32-key block
  constexpr int kBatch = 4;
  constexpr int kBatches = 2 * kSteps / kBatch;
  const int lane = threadIdx.x & 63, c = lane & 31, hh = lane >> 5;
  const char* base = sK + K16::at(c, hh * 16);
  half8 kf[2][kBatch];
  auto load = [&](int bt, half8* dst) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int step = bt * kBatch + i, kb = step / kSteps, kk = step % kSteps;
      dst[i] = *reinterpret_cast<const half8*>(base + K16::at(kb * 32, kk * 32));
    }
  };
  acc[0] = (float16v){};
  acc[1] = (float16v){};
  load(0, kf[0]);
#pragma unroll
  for (int bt = 0; bt < kBatches; ++bt) {
    TM_FENCE();
    if (bt + 1 < kBatches) load(bt + 1, kf[(bt + 1) & 1]);
    TM_FENCE();
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int step = bt * kBatch + i, kb = step / kSteps, kk = step % kSteps;
      acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[bt & 1][i], qf[kk], acc[kb], 0, 0, 0);
    }
  }
  TM_FENCE();
}

// FP8 (E4M3) path of the same block: S^T = K_f8 . Q_f8^T, fp32 accumulation
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales).  A lane holds
// 32 consecutive codes of its row in each 64-wide step, for K and Q alike.
template <int D>
__device__ inline void qk_tile_f8(const char* sK, const int8v* qc, float16v acc[2]) {
  using K8 = typename Tile<D>::K8;
  constexpr int kSteps = D / 64;               // per 32-key block
  const int lane = threadIdx.x & 63, c = lane & 31, hh = lane >> 5;
  const char* base = sK + K8::at(c, hh * 32);
  int8v kf[2 * kSteps];
#pragma unroll
  for (int step = 0; step < 2 * kSteps; ++step) {
    const int kb = step / kSteps, kk = step % kSteps;
    const char* p = base + K8::at(kb * 32, kk * 64);
    const int4v lo = *reinterpret_cast<const int4v*>(p);
    const int4v hi = *reinterpret_cast<const int4v*>(p + 16);
    kf[step] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  TM_FENCE();
  acc[0] = (float16v){};
  acc[1] = (float16v){};
#pragma unroll
  for (int step = 0; step < 2 * kSteps; ++step) {
    const int kb = step / kSteps, kk = step % kSteps;
    acc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[step], qc[kk], acc[kb], 0, 0, 0, 0x7f7f7f7f,
                                                            0, 0x7f7f7f7f);
  }
  TM_FENCE();
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

// The work unit's Q block quantised in registers ([Digest, method]: Q blocks
// of 128 x d, s = absmax / 127, the quantiser's arithmetic element for
// element).  qf holds this lane's fp16 fragments (zeros for rows past the
// sequence end, which leave the absmax unchanged); red is 4 floats of LDS.
// Codes are made in the fp16 fragment order (lane half hh holds dims
// 16 kk + 8 hh + 0..7) and moved into the INT8 one (dims 32 kk + 16 hh +
// 0..15) by one exchange per dword with lane l ^ 32.  Returns the scale.
template <int D>
__device__ inline float quantize_q_inline(const half8* qf, int4v* qb, float* red, int w, float* amax_out) {
  const int lane = threadIdx.x & 63;
  half2v m2[4] = {};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const half2v p = {qf[kk][2 * j], qf[kk][2 * j + 1]};
      m2[j] = __builtin_elementwise_max(m2[j], __builtin_elementwise_abs(p));
    }
  m2[0] = __builtin_elementwise_max(__builtin_elementwise_max(m2[0], m2[1]), __builtin_elementwise_max(m2[2], m2[3]));
  float amax = fmaxf((float)m2[0][0], (float)m2[0][1]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if (lane == 0) red[w] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  *amax_out = amax;
  const float s = __fdiv_rn(amax, 127.0f);
  const float rs = amax > 0.f ? __fdiv_rn(1.0f, s) : 0.f;
  // Straight-line pass: t = fl(x * rs + 1.5 * 2^23) rounds the exact product
  // p = x * rs (|p| <= 127 + tiny) half-to-even to the integer t - 1.5 * 2^23,
  // whose low byte is the low byte of t's bits; e = p - code (to 2^-25).  p
  // lies within 1.2e-5 of fl(x / s) (rs's rounding plus half an ulp of the
  // quotient), so the code equals round-half-even(fl(x / s)) unless |e| >
  // 0.5 - 2^-16.  A word of four codes with such an element in any lane is
  // redone across the wave with quant_code_i8, element for element.
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
  uint32_t cw[D / 16][2];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t b[4];
      float emax = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = (float)qf[kk][4 * h + j];
        const float t = __builtin_fmaf(x, rs, kMagic);
        const float e = __builtin_fmaf(x, rs, kMagic - t);
        emax = fmaxf(emax, __builtin_fabsf(e));
        b[j] = __builtin_bit_cast(uint32_t, t);
      }
      uint32_t word = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u) | __builtin_amdgcn_perm(b[3], b[2], 0x04000c0cu);
      if (__builtin_amdgcn_ballot_w64(emax > 0.5f - 0x1p-16f)) {
        word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          word |= (uint32_t)(quant_code_i8((float)qf[kk][4 * h + j], rs, s) & 0xff) << (8 * j);
      }
      cw[kk][h] = word;
    }
  // Lanes 32..63 of the first operand trade places with lanes 0..31 of the
  // second: the low half keeps its own dims 32 kk2 + 0..7 and receives the
  // high half's 8..15; the high half receives the low half's 16..23 and keeps
  // its own 24..31.
#pragma unroll
  for (int kk2 = 0; kk2 < D / 32; ++kk2) {
    const auto r0 = __builtin_amdgcn_permlane32_swap(cw[2 * kk2][0], cw[2 * kk2 + 1][0], false, false);
    const auto r1 = __builtin_amdgcn_permlane32_swap(cw[2 * kk2][1], cw[2 * kk2 + 1][1], false, false);
    qb[kk2] = (int4v){(int)r0[0], (int)r1[0], (int)r0[1], (int)r1[1]};
  }
  return s;
}

// The same Q block's E4M3 codes ([Digest, method] blocks; s = fl(a / 448),
// code = E4M3 round-half-even of fl(x / s), as the FP8 quantiser), from the
// block absmax a.  fl(x / s) lies strictly between x * rl and x * rh, where
// rl and rh are fl(1 / s) nudged down and up by 2^-21 (each product is then
// within 2^-22 of x / s on its own side), and the conversion is monotone: where
// both products give the same code, so does fl(x / s).  A word of four codes
// with any other element in any lane is redone across the wave with the IEEE
// quotient (exact E4M3 ties are common: fl(x / s) lands on a midpoint for
// about one element in a thousand of random blocks).  Codes are made in the
// fp16 fragment order and exchanged with lane l ^ 32 into the FP8 one (lane
// half hh holds dims 64 kk + 32 hh + 0..31).  Returns the scale.
template <int D>
__device__ inline float quantize_q_inline_f8(const half8* qf, int8v* qc, float amax) {
  const float s = __fdiv_rn(amax, 448.0f);
  const float rs = amax > 0.f ? __fdiv_rn(1.0f, s) : 0.f;
  const float rl = rs * (1.0f - 0x1p-21f), rh = rs * (1.0f + 0x1p-21f);
  uint32_t cw[D / 16][2];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float lo[4], hi[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = (float)qf[kk][4 * h + j];
        lo[j] = x * rl;
        hi[j] = x * rh;
      }
      int cl = __builtin_amdgcn_cvt_pk_fp8_f32(lo[0], lo[1], 0, false);
      cl = __builtin_amdgcn_cvt_pk_fp8_f32(lo[2], lo[3], cl, true);
      int ch = __builtin_amdgcn_cvt_pk_fp8_f32(hi[0], hi[1], 0, false);
      ch = __builtin_amdgcn_cvt_pk_fp8_f32(hi[2], hi[3], ch, true);
      if (__builtin_amdgcn_ballot_w64(cl != ch)) {
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = amax > 0.f ? __fdiv_rn((float)qf[kk][4 * h + j], s) : 0.f;
        cl = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        cl = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], cl, true);
      }
      cw[kk][h] = (uint32_t)cl;
    }
  // Group m (8 dims) of the FP8 fragment kk: the low lane half takes its own
  // fp16 groups 4kk, 4kk+1 and the high half's same ones; the high half the
  // low half's 4kk+2, 4kk+3 and its own.
#pragma unroll
  for (int kk = 0; kk < D / 64; ++kk) {
    uint32_t g[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const auto a = __builtin_amdgcn_permlane32_swap(cw[4 * kk][h], cw[4 * kk + 2][h], false, false);
      const auto b = __builtin_amdgcn_permlane32_swap(cw[4 * kk + 1][h], cw[4 * kk + 3][h], false, false);
      g[0 + h] = a[0];
      g[2 + h] = a[1];
      g[4 + h] = b[0];
      g[6 + h] = b[1];
    }
    qc[kk] = (int8v){(int)g[0], (int)g[1], (int)g[2], (int)g[3], (int)g[4], (int)g[5], (int)g[6], (int)g[7]};
  }
  return s;
}

// --------------------------------------------------------------------------
// Fused mixed-precision prefill.  One workgroup = one work unit (sequence,
// query head, 128-row query tile); wave w owns queries 32w .. 32w+31.
// Per legal key tile: routing bit lookup ([Map, hot loop]: shift and mask),
// QK^T on the routed path, rescale into the common score domain ([Explainer,
// 第三步]), causal/sequence-end mask, shared online softmax, P.V in FP16
// ([Digest, method]).  Tile t+1 streams into the other LDS buffer while tile
// t is computed; one barrier per tile.  Tiles before the row's diagonal need
// no mask and run in a separate loop.
//
// Online softmax in the log2 domain: x = S * log2(e).  The running maximum m
// is raised only when a row's tile maximum exceeds it by more than kLazy
// (then O and l are rescaled); otherwise P = 2^(x - m) <= 2^kLazy = 16384, which
// fp16 holds exactly as well as any P <= 1.  O / l does not depend on the m
// chosen, so this changes rounding only.
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
  // third path (FP8): codes, scales and the FP8 routing words (unused by the
  // two-path kernel)
  const uint8_t* qf8;
  const uint8_t* kf8;
  const float* qsf8;
  const float* ksf8;
  const uint64_t* wordsf8;
  int32_t hq, hkv, tq, tk;
};

constexpr float kLazy = 14.0f;

template <int D>
struct RowState {
  float m, lsum;
  float16v o[D / 32];
};

// code: 0 FP16, 1 INT8, 2 FP8 (the FP8 arm exists only with kThree).  With
// kMasked, `cross` (wave-uniform) says whether some key of the tile lies past
// some query's diagonal or the sequence end; only then is the mask applied.
template <int D, bool kMasked, bool kThree>
__device__ __forceinline__ void tile_step(const char* buf, int code, float f_i8, float f16s, const half8* qf,
                                          const int4v* qb, const int8v* qc, float f_f8, RowState<D>& st,
                                          int k0, int qi, int L, bool cross) {
  const int lane = threadIdx.x & 63, hh = lane >> 5;
  float16v accv[2];
  float f;
  if (kThree && code == 2) {
    qk_tile_f8<D>(buf, qc, accv);
    f = f_f8;
  } else if (code) {
    int16v acc[2];
    qk_tile_i8<D>(buf, qb, acc);
    f = f_i8;
    // exact: |acc| <= 127^2 d < 2^24
    accv[0] = __builtin_convertvector(acc[0], float16v);
    accv[1] = __builtin_convertvector(acc[1], float16v);
  } else {
    qk_tile_f16<D>(buf, qf, accv);
    f = f16s;
  }
  float accf[2][16];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) accf[kb][i] = accv[kb][i];
  // Causal / sequence-end mask, independent of the routing bit: key
  // k0 + 4 hh + c (c a compile-time offset) is visible to query qi when
  // c <= min(qi, L - 1) - k0 - 4 hh; the others become -inf here and give
  // P = 2^-inf = 0 below.  That needs a positive factor.  The factor is zero
  // only for an all-zero Q or K block (a nonzero block scale is at least
  // 2^-24 / 448, so no product of two underflows), whose codes and scores
  // are all zero: the least normal float in its place leaves them zero.
  if (kMasked && cross) {
    const int lim = min(qi, L - 1) - k0 - hh * 4;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kb * 32 + (i >> 2) * 8 + (i & 3) > lim) accf[kb][i] = -INFINITY;
    f = f > 0.f ? f : FLT_MIN;
  }
  // The vector-ALU softmax runs at raised wave priority: the sooner it
  // finishes, the sooner this wave's P.V matrix instructions are ready to
  // fill the matrix pipe beside the other wave's.
  __builtin_amdgcn_s_setprio(1);
  // Row maximum of the raw accumulators (f >= 0 preserves the order).
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, accf[kb][i]);
  mx = max_with_other_half(mx);
  mx = (mx == -INFINITY) ? -INFINITY : mx * f;
  // Wave-uniform: when some row's maximum has outgrown m by more than kLazy,
  // the wave rescales O anyway, so every row whose tile maximum exceeds its m
  // takes it now (fewer later rescales; P <= 2^kLazy still holds).
  if (__builtin_amdgcn_ballot_w64(mx > st.m + kLazy)) {
    const float mnew = fmaxf(st.m, mx);
    const float alpha = mnew == st.m ? 1.0f : __builtin_amdgcn_exp2f(st.m - mnew);
    st.m = mnew;
    st.lsum *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.o[db] *= alpha;
  }
  const float negm = -st.m;
  uint32_t pw[2][8];
  float psum = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(accf[kb][2 * i], f, negm));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(accf[kb][2 * i + 1], f, negm));
      const half2v pk = {(_Float16)e0, (_Float16)e1};
      psum = __builtin_amdgcn_fdot2(pk, (half2v){(_Float16)1.0f, (_Float16)1.0f}, psum, false);
      pw[kb][i] = __builtin_bit_cast(uint32_t, pk);
    }
  st.lsum += psum;
  __builtin_amdgcn_s_setprio(0);

  // O^T += V^T . P^T (fp16 operands, fp32 accumulation).  V fragments come
  // transposed from LDS: a 16-lane group gives lane i the column i of 4
  // consecutive rows.
  using VL = typename Tile<D>::V;
  const int j = lane & 15, sub = (lane >> 4) & 1;
  // rows ks*16 + x (+8), x = hh*4 + j/4 < 8: window and slot split into a
  // lane part and a compile-time part (the window count is 16 or 8).
  const char* vbase = buf + Tile<D>::kKRegion + VL::at(hh * 4 + (j >> 2), (sub * 16 + 4 * (j & 3)) * 2);
  half8 vf[2][D / 32];
  auto load_v = [&](int ks, half8* dst) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const char* a0 = vbase + VL::at(ks * 16, db * 64);
      const char* a1 = vbase + VL::at(ks * 16 + 8, db * 64);
      // Whole-vector casts: element-wise extraction of the transposed
      // read's result is mis-assembled by this compiler.
      const half4 lo = __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(short4v, a0)));
      const half4 hi = __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(short4v, a1)));
      dst[db] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  load_v(0, vf[0]);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    TM_FENCE();
    if (ks + 1 < 4) load_v(ks + 1, vf[(ks + 1) & 1]);
    TM_FENCE();
    const int kb = ks >> 1, hf = ks & 1;
    const half8 pf = __builtin_bit_cast(half8, (uint4){pw[kb][hf * 4 + 0], pw[kb][hf * 4 + 1],
                                                       pw[kb][hf * 4 + 2], pw[kb][hf * 4 + 3]});
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[ks & 1][db], pf, st.o[db], 0, 0, 0);
  }
  TM_FENCE();
}

// kThree adds the FP8 path: a second word per (KV head, row) marks FP8
// groups (never also INT8); without it the kernel is the two-path one.
// kQInline: the unit's Q block is quantised in the prologue (INT8, and FP8
// with kThree) instead of read from the quantisers' output (a.qi8, a.qs,
// a.qf8, a.qsf8 unused).
template <int D, bool kThree, bool kQInline = false>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  using T = Tile<D>;

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
  const uint64_t wordf = kThree ? a.wordsf8[(size_t)kv * a.tq + qt_off + row] : 0ull;

  const int tid = threadIdx.x, lane = tid & 63, c = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = q0 + 32 * w + c;  // this lane's query (sequence-local)
  const bool qvalid = qi < L;

  const int s16 = a.hkv * D * 2, s8 = a.hkv * D;  // bytes between consecutive K/V rows
  const char* kseq = reinterpret_cast<const char*>(a.k + ((size_t)start * a.hkv + kv) * D);
  const char* k8seq = reinterpret_cast<const char*>(a.ki8 + ((size_t)start * a.hkv + kv) * D);
  const char* vseq = reinterpret_cast<const char*>(a.v + ((size_t)start * a.hkv + kv) * D);
  const char* kf8seq = kThree ? reinterpret_cast<const char*>(a.kf8 + ((size_t)start * a.hkv + kv) * D) : nullptr;
  const int lo16 = T::K16::lane_src(lane, s16), lo8 = T::K8::lane_src(lane, s8);
  const int lov = T::V::lane_src(lane, s16);

  // Routing code of tile t's group G = t / g (tracked incrementally): 1 INT8
  // when (word >> G) & 1, else 2 FP8 when (wordf >> G) & 1, else 0 FP16.
  int grp = 0, in_grp = 0;  // group of the current tile, position in it
  auto code_of = [&](int G) {
    return ((word >> G) & 1ull) ? 1 : (kThree && ((wordf >> G) & 1ull)) ? 2 : 0;
  };
  const unsigned lds0 = __builtin_amdgcn_readfirstlane((unsigned)(size_t)LDS_PTR(char, smem));
  auto issue = [&](int t, int code, char* buf) {
    const int nvalid = min(kBlockN, L - t * kBlockN);
    if (nvalid == kBlockN) {  // a whole tile: the lean form
      const unsigned lb = lds0 + (unsigned)(buf - smem);
      if (code == 1) T::K8::issue_full(lb, k8seq + (size_t)t * kBlockN * s8, s8, w, lo8);
      else if (kThree && code == 2) T::K8::issue_full(lb, kf8seq + (size_t)t * kBlockN * s8, s8, w, lo8);
      else T::K16::issue_full(lb, kseq + (size_t)t * kBlockN * s16, s16, w, lo16);
      T::V::issue_full(lb + T::kKRegion, vseq + (size_t)t * kBlockN * s16, s16, w, lov);
      return;
    }
    if (code == 1) T::K8::issue(buf, k8seq + (size_t)t * kBlockN * s8, s8, nvalid, w, lane, lo8);
    else if (kThree && code == 2) T::K8::issue(buf, kf8seq + (size_t)t * kBlockN * s8, s8, nvalid, w, lane, lo8);
    else T::K16::issue(buf, kseq + (size_t)t * kBlockN * s16, s16, nvalid, w, lane, lo16);
    T::V::issue(buf + T::kKRegion, vseq + (size_t)t * kBlockN * s16, s16, nvalid, w, lane, lov);
  };
  issue(0, code_of(0), smem);

  half8 qf[D / 16];
  int4v qb[D / 32];
  if (!kQInline) {
    load_q<D>(a.q + ((size_t)(start + qi) * a.hq + head) * D,
              a.qi8 + ((size_t)(start + qi) * a.hq + head) * D, qvalid, qf, qb);
  } else {
    // the fp16 fragments only (quantised below), in flight with the first tile
    const _Float16* qrow = a.q + ((size_t)(start + qi) * a.hq + head) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      half8 v = {};
      if (qvalid) v = *reinterpret_cast<const half8*>(qrow + kk * 16 + (lane >> 5) * 8);
      qf[kk] = v;
    }
  }
  int8v qc[kThree ? D / 64 : 1];  // FP8 query codes: 32 per lane per 64-wide step
  if (kThree && !kQInline) {
    const uint8_t* qrow = a.qf8 + ((size_t)(start + qi) * a.hq + head) * D;
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) {
      int4v lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
      if (qvalid) {
        lo = *reinterpret_cast<const int4v*>(qrow + kk * 64 + (lane >> 5) * 32);
        hi = *reinterpret_cast<const int4v*>(qrow + kk * 64 + (lane >> 5) * 32 + 16);
      }
      qc[kk] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
  // The row's key-tile scales go through LDS (1024 tiles per chunk): a scalar
  // load per tile would make every later lgkmcnt wait include its memory
  // latency.  The first chunk's (and Q's scales, when they come from the
  // quantiser) are loaded here, with Q's values, and stored below: staged
  // after the Q block they had cost each work unit one more memory latency.
  const float* kscale = a.ks + (size_t)kv * a.tk + kt_off;
  float* sks = reinterpret_cast<float*>(smem + 2 * T::kBuf);
  const float* kscalef = kThree ? a.ksf8 + (size_t)kv * a.tk + kt_off : nullptr;
  float* sksf = sks + T::kScales;  // (FP8 scales, three-path kernel only)
  constexpr int kPre = T::kScales / kThreads;
  const int npre = min(T::kScales, last_tile + 1);
  float scp[kPre], scfp[kThree ? kPre : 1];
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    const int i = tid + j * kThreads;
    if (i < npre) {
      scp[j] = kscale[i];
      if (kThree) scfp[j] = kscalef[i];
    }
  }
  const float sq_ld = kQInline ? 0.f : load_uniform(a.qs + (size_t)head * a.tq + qt_off + row);
  const float sqf_ld = (kQInline || !kThree) ? 0.f : load_uniform(a.qsf8 + (size_t)head * a.tq + qt_off + row);
  // Let the compiler see the query loads complete here: it does not count the
  // asm-issued tile loads, so a wait it placed later for these would also
  // wait for every tile load in flight.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  float sq, sqf = 0.f;
  if (kQInline) {
    // past the key-tile scales (and the FP8 ones): those are staged below
    // while slower waves may still read the exchanged maxima
    float* red = reinterpret_cast<float*>(smem + 2 * T::kBuf) + (kThree ? 2 : 1) * T::kScales;
    float amax;
    const float s = quantize_q_inline<D>(qf, qb, red, w, &amax);
    sq = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, s)));
    if (kThree) {
      const float sf = quantize_q_inline_f8<D>(qf, qc, amax);
      sqf = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sf)));
    }
  } else {
    sq = sq_ld;
    sqf = sqf_ld;
  }
  const float inv_sqrt_d = (float)(1.0 / std::sqrt((double)D));
  const float scale16 = inv_sqrt_d * kLog2e;
  // later chunks (rows of more than 1024 key tiles)
  auto stage_scales = [&](int t0) {
    const int n = min(T::kScales, last_tile + 1 - t0);
    for (int i = tid; i < n; i += kThreads) sks[i] = kscale[t0 + i];
    if (kThree)
      for (int i = tid; i < n; i += kThreads) sksf[i] = kscalef[t0 + i];
  };
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    const int i = tid + j * kThreads;
    if (i < npre) {
      sks[i] = scp[j];
      if (kThree) sksf[i] = scfp[j];
    }
  }

  RowState<D> st;
  st.m = -INFINITY;
  st.lsum = 0.f;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) st.o[i] = (float16v){};

  // One pipelined step: wait for tile t, start tile t+1, compute tile t.
  auto step = [&](int t, auto masked) {
    char* buf = smem + (t & 1) * T::kBuf;
    const int code = code_of(grp);
    const int ngrp = (in_grp + 1 == g) ? grp + 1 : grp;
    in_grp = (in_grp + 1 == g) ? 0 : in_grp + 1;
    wait_tile_loads();
    __syncthreads();  // tile t visible; everyone is done with tile t-1's buffer
    if (t > 0 && (t & (T::kScales - 1)) == 0) {  // next chunk of scales
      stage_scales(t);
      __syncthreads();
    }
    if (t < last_tile) issue(t + 1, code_of(ngrp), smem + ((t + 1) & 1) * T::kBuf);
    grp = ngrp;
    const float f_i8 = (sq * sks[t & (T::kScales - 1)]) * inv_sqrt_d * kLog2e;
    const float f_f8 = kThree ? (sqf * sksf[t & (T::kScales - 1)]) * inv_sqrt_d * kLog2e : 0.f;
    const int k0 = t * kBlockN;
    if constexpr (!decltype(masked)::value) {
      tile_step<D, false, kThree>(buf, code, f_i8, scale16, qf, qb, qc, f_f8, st, k0, qi, L, false);
    } else {
      // Wave-uniform: a tile none of whose keys any of the wave's queries
      // sees (or a wave past the sequence end) adds P = 0 and is skipped; a
      // tile all of whose keys every query of the wave sees skips the mask
      // (the same code with a branch, not a second copy of the tile step:
      // two copies in this loop push the kernel past 256 registers).
      const int qlo = q0 + 32 * w, qhi = min(qlo + 31, L - 1);
      if (k0 <= qhi && qlo < L) {
        const bool cross = k0 + kBlockN - 1 > qlo || k0 + kBlockN > L;
        tile_step<D, true, kThree>(buf, code, f_i8, scale16, qf, qb, qc, f_f8, st, k0, qi, L, cross);
      }
    }
  };
  // Tiles t < 2 row lie entirely below the diagonal of every query of the
  // work unit and inside the sequence: no mask.  The rest (the diagonal
  // tiles and a partial last tile) run in a second loop, where each wave
  // takes the mask only on the tiles that cross its own queries' diagonal.
  int t = 0;
  for (; t < 2 * row; ++t) step(t, std::false_type{});
  for (; t <= last_tile; ++t) step(t, std::true_type{});

  // Epilogue: O = acc / l, fp16 round-to-nearest-even.
  const int hh = lane >> 5;
  const float ltot = sum_with_other_half(st.lsum);
  const float inv = 1.0f / ltot;
  if (qvalid) {
    _Float16* orow = a.out + ((size_t)(start + qi) * a.hq + head) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        half4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = (_Float16)(st.o[db][i4 * 4 + e] * inv);
        *reinterpret_cast<half4*>(orow + db * 32 + i4 * 8 + hh * 4) = h;
      }
  }
}

// Int32 accumulator of one INT8 score tile, through the kernel's own tile
// loader and qk_tile_i8 routine.
template <int D>
__global__ __launch_bounds__(kThreads) void debug_qk_i32_kernel(const int32_t* plan, const int8_t* qi8,
                                                                const int8_t* ki8, int seq, int head,
                                                                int row, int t, int32_t* acc_out) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(1024))) char sK[T::K8::kBytes];
  const int hq = plan[kHq], hkv = plan[kHkv];
  const int32_t* rec = plan + kHeaderLen + seq * kSeqStride;
  const int start = rec[kSeqStart], L = rec[kSeqLen];
  const int kv = head / (hq / hkv);
  const int tid = threadIdx.x, lane = tid & 63, c = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = row * kBlockM + 32 * w + c;
  const int k0 = t * kBlockN;
  const int nvalid = min(kBlockN, L - k0);
  const int s8 = hkv * D;
  T::K8::issue(sK, ki8 + ((size_t)(start + k0) * hkv + kv) * D, s8, nvalid, w, lane,
               T::K8::lane_src(lane, s8));
  int4v qb[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    int4v v = {0, 0, 0, 0};
    if (qi < L)
      v = *reinterpret_cast<const int4v*>(qi8 + ((size_t)(start + qi) * hq + head) * D + kk * 32 + hh * 16);
    qb[kk] = v;
  }
  wait_tile_loads();
  __syncthreads();
  int16v acc[2];
  qk_tile_i8<D>(sK, qb, acc);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kb * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
      // keys past the sequence end hold a repeated row in LDS: report 0
      acc_out[(32 * w + c) * kBlockN + key] = (k0 + key < L) ? acc[kb][i] : 0;
    }
}

// Fp32 accumulator of one FP8 score tile (the E4M3 codes' products summed by
// the matrix instruction, no scale applied), through the kernel's own tile
// loader and qk_tile_f8 routine.
template <int D>
__global__ __launch_bounds__(kThreads) void debug_qk_f8_kernel(const int32_t* plan, const uint8_t* qf8,
                                                               const uint8_t* kf8, int seq, int head, int row,
                                                               int t, float* acc_out) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(1024))) char sK[T::K8::kBytes];
  const int hq = plan[kHq], hkv = plan[kHkv];
  const int32_t* rec = plan + kHeaderLen + seq * kSeqStride;
  const int start = rec[kSeqStart], L = rec[kSeqLen];
  const int kv = head / (hq / hkv);
  const int tid = threadIdx.x, lane = tid & 63, c = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = row * kBlockM + 32 * w + c;
  const int k0 = t * kBlockN;
  const int nvalid = min(kBlockN, L - k0);
  const int s8 = hkv * D;
  T::K8::issue(sK, kf8 + ((size_t)(start + k0) * hkv + kv) * D, s8, nvalid, w, lane, T::K8::lane_src(lane, s8));
  int8v qc[D / 64];
#pragma unroll
  for (int kk = 0; kk < D / 64; ++kk) {
    int4v lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
    if (qi < L) {
      const uint8_t* qrow = qf8 + ((size_t)(start + qi) * hq + head) * D + kk * 64 + hh * 32;
      lo = *reinterpret_cast<const int4v*>(qrow);
      hi = *reinterpret_cast<const int4v*>(qrow + 16);
    }
    qc[kk] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  wait_tile_loads();
  __syncthreads();
  float16v acc[2];
  qk_tile_f8<D>(sK, qc, acc);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kb * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
      acc_out[(32 * w + c) * kBlockN + key] = (k0 + key < L && qi < L) ? acc[kb][i] : 0.f;
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

namespace tilemix {

int check_plans(const int32_t* plan_h, const int32_t* plan_d) {
  int rc = check_plan(plan_h);
  if (rc) return rc;
  if ((rc = check_dev_ptr(plan_d, "plan_d", true))) return rc;
#ifdef TILEMIX_DEBUG_PLAN
  int32_t head[kHeaderLen];
  hipError_t e = hipMemcpy(head, plan_d, sizeof head, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "reading back plan_d");
  for (int i = 0; i < kHeaderLen; ++i)
    if (head[i] != plan_h[i]) return fail(TILEMIX_EINVAL, "plan_d is not the device copy of plan_h (field %d)", i);
#endif
  return TILEMIX_OK;
}

}  // namespace tilemix

extern "C" {

int tilemix_quantize_qk(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                        const void* k_f16, int8_t* q_i8, int8_t* k_i8, float* q_scale,
                        float* k_scale, void* hip_stream) {
  clear_error();
  int rc = check_plans(plan_h, plan_d);
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
  int rc = check_plans(plan_h, plan_d);
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
  a.qf8 = nullptr;
  a.kf8 = nullptr;
  a.qsf8 = nullptr;
  a.ksf8 = nullptr;
  a.wordsf8 = nullptr;
  a.hq = plan_h[kHq];
  a.hkv = plan_h[kHkv];
  a.tq = plan_h[kTotalQTiles];
  a.tk = plan_h[kTotalKTiles];
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const unsigned grid = (unsigned)plan_h[kNumItems];
  if (plan_h[kHeadDim] == 64)
    hipLaunchKernelGGL((prefill_kernel<64, false>), dim3(grid), dim3(kThreads), Tile<64>::kLds, st, a);
  else
    hipLaunchKernelGGL((prefill_kernel<128, false>), dim3(grid), dim3(kThreads), Tile<128>::kLds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return TILEMIX_OK;
}

int tilemix_quantize_k(const int32_t* plan_h, const int32_t* plan_d, const void* k_f16, int8_t* k_i8,
                       float* k_scale, void* hip_stream) {
  clear_error();
  int rc = check_plans(plan_h, plan_d);
  if (rc) return rc;
  const bool any = plan_h[kTotalTokens] > 0;
  if ((rc = check_dev_ptr(plan_d, "plan_d", true)) || (rc = check_dev_ptr(k_f16, "k_f16", any)) ||
      (rc = check_dev_ptr(k_i8, "k_i8", any)) || (rc = check_dev_ptr(k_scale, "k_scale", any)))
    return rc;
  if (!any) return TILEMIX_OK;
  QuantArgs a;
  a.plan = plan_d;
  a.q = nullptr;  // key blocks only
  a.k = static_cast<const _Float16*>(k_f16);
  a.qi8 = nullptr;
  a.ki8 = k_i8;
  a.qs = nullptr;
  a.ks = k_scale;
  a.hq = plan_h[kHq];
  a.hkv = plan_h[kHkv];
  a.batch = plan_h[kBatch];
  a.tq = plan_h[kTotalQTiles];
  a.tk = plan_h[kTotalKTiles];
  // grid: (key tiles of the longest sequence x KV heads, sequences)
  int64_t max_tn = 0;
  for (int32_t s = 0; s < a.batch; ++s) {
    const int64_t L = plan_h[kHeaderLen + s * kSeqStride + kSeqLen];
    max_tn = std::max<int64_t>(max_tn, (L + kBlockN - 1) / kBlockN);
  }
  const int64_t gx = max_tn * a.hkv;
  if (gx > 0x7fffffff || a.batch > 65535) return fail(TILEMIX_EINVAL, "batch too large for one launch");
  if ((int64_t)a.hkv * plan_h[kHeadDim] * 2 * kBlockN > 0x7fffffff)
    return fail(TILEMIX_EINVAL, "%d KV heads: a 64-row key block spans more than 2 GiB", a.hkv);
  if (gx == 0) return TILEMIX_OK;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const dim3 grid((unsigned)gx, (unsigned)a.batch);
  if (plan_h[kHeadDim] == 64)
    hipLaunchKernelGGL(quantize_k_kernel<64>, grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(quantize_k_kernel<128>, grid, dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "quantize_k launch");
  return TILEMIX_OK;
}

int tilemix_prefill_varlen_qinline(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                                   const void* k_f16, const void* v_f16, const int8_t* k_i8,
                                   const float* k_scale, const uint64_t* words_d, void* out_f16,
                                   void* hip_stream) {
  clear_error();
  int rc = check_plans(plan_h, plan_d);
  if (rc) return rc;
  const bool any = plan_h[kNumItems] > 0;
  if ((rc = check_dev_ptr(plan_d, "plan_d", true)) || (rc = check_dev_ptr(q_f16, "q_f16", any)) ||
      (rc = check_dev_ptr(k_f16, "k_f16", any)) || (rc = check_dev_ptr(v_f16, "v_f16", any)) ||
      (rc = check_dev_ptr(k_i8, "k_i8", any)) || (rc = check_dev_ptr(k_scale, "k_scale", any)) ||
      (rc = check_dev_ptr(words_d, "words_d", any)) || (rc = check_dev_ptr(out_f16, "out_f16", any)))
    return rc;
  if (!any) return TILEMIX_OK;
  PrefillArgs a;
  a.plan = plan_d;
  a.q = static_cast<const _Float16*>(q_f16);
  a.k = static_cast<const _Float16*>(k_f16);
  a.v = static_cast<const _Float16*>(v_f16);
  a.qi8 = nullptr;  // Q is quantised in the kernel
  a.ki8 = k_i8;
  a.qs = nullptr;
  a.ks = k_scale;
  a.words = words_d;
  a.out = static_cast<_Float16*>(out_f16);
  a.qf8 = nullptr;
  a.kf8 = nullptr;
  a.qsf8 = nullptr;
  a.ksf8 = nullptr;
  a.wordsf8 = nullptr;
  a.hq = plan_h[kHq];
  a.hkv = plan_h[kHkv];
  a.tq = plan_h[kTotalQTiles];
  a.tk = plan_h[kTotalKTiles];
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const unsigned grid = (unsigned)plan_h[kNumItems];
  if (plan_h[kHeadDim] == 64)
    hipLaunchKernelGGL((prefill_kernel<64, false, true>), dim3(grid), dim3(kThreads), Tile<64>::kLdsQ, st, a);
  else
    hipLaunchKernelGGL((prefill_kernel<128, false, true>), dim3(grid), dim3(kThreads), Tile<128>::kLdsQ, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "prefill_qinline launch");
  return TILEMIX_OK;
}

int tilemix_quantize_qk_fp8(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                            const void* k_f16, uint8_t* q_f8, uint8_t* k_f8, float* q_scale_f8,
                            float* k_scale_f8, void* hip_stream) {
  clear_error();
  int rc = check_plans(plan_h, plan_d);
  if (rc) return rc;
  const bool any = plan_h[kTotalTokens] > 0;
  if ((rc = check_dev_ptr(plan_d, "plan_d", true)) || (rc = check_dev_ptr(q_f16, "q_f16", any)) ||
      (rc = check_dev_ptr(k_f16, "k_f16", any)) || (rc = check_dev_ptr(q_f8, "q_f8", any)) ||
      (rc = check_dev_ptr(k_f8, "k_f8", any)) || (rc = check_dev_ptr(q_scale_f8, "q_scale_f8", any)) ||
      (rc = check_dev_ptr(k_scale_f8, "k_scale_f8", any)))
    return rc;
  if (!any) return TILEMIX_OK;
  QuantFp8Args a;
  a.plan = plan_d;
  a.q = static_cast<const _Float16*>(q_f16);
  a.k = static_cast<const _Float16*>(k_f16);
  a.qf8 = q_f8;
  a.kf8 = k_f8;
  a.qs = q_scale_f8;
  a.ks = k_scale_f8;
  a.hq = plan_h[kHq];
  a.hkv = plan_h[kHkv];
  a.batch = plan_h[kBatch];
  a.tq = plan_h[kTotalQTiles];
  a.tk = plan_h[kTotalKTiles];
  const int64_t blocks = (int64_t)a.tq * a.hq + (int64_t)a.tk * a.hkv;
  if (blocks > 0x7fffffff) return fail(TILEMIX_EINVAL, "batch too large for one launch");
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (plan_h[kHeadDim] == 64)
    hipLaunchKernelGGL(quantize_qk_fp8_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(quantize_qk_fp8_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "fp8 quantize launch");
  return TILEMIX_OK;
}

int tilemix_prefill_varlen3(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                            const void* k_f16, const void* v_f16, const int8_t* q_i8, const int8_t* k_i8,
                            const float* q_scale, const float* k_scale, const uint8_t* q_f8,
                            const uint8_t* k_f8, const float* q_scale_f8, const float* k_scale_f8,
                            const uint64_t* words_i8_d, const uint64_t* words_f8_d, void* out_f16,
                            void* hip_stream) {
  clear_error();
  int rc = check_plans(plan_h, plan_d);
  if (rc) return rc;
  const bool any = plan_h[kNumItems] > 0;
  if ((rc = check_dev_ptr(plan_d, "plan_d", true)) || (rc = check_dev_ptr(q_f16, "q_f16", any)) ||
      (rc = check_dev_ptr(k_f16, "k_f16", any)) || (rc = check_dev_ptr(v_f16, "v_f16", any)) ||
      (rc = check_dev_ptr(q_i8, "q_i8", any)) || (rc = check_dev_ptr(k_i8, "k_i8", any)) ||
      (rc = check_dev_ptr(q_scale, "q_scale", any)) || (rc = check_dev_ptr(k_scale, "k_scale", any)) ||
      (rc = check_dev_ptr(q_f8, "q_f8", any)) || (rc = check_dev_ptr(k_f8, "k_f8", any)) ||
      (rc = check_dev_ptr(q_scale_f8, "q_scale_f8", any)) || (rc = check_dev_ptr(k_scale_f8, "k_scale_f8", any)) ||
      (rc = check_dev_ptr(words_i8_d, "words_i8_d", any)) || (rc = check_dev_ptr(words_f8_d, "words_f8_d", any)) ||
      (rc = check_dev_ptr(out_f16, "out_f16", any)))
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
  a.words = words_i8_d;
  a.out = static_cast<_Float16*>(out_f16);
  a.qf8 = q_f8;
  a.kf8 = k_f8;
  a.qsf8 = q_scale_f8;
  a.ksf8 = k_scale_f8;
  a.wordsf8 = words_f8_d;
  a.hq = plan_h[kHq];
  a.hkv = plan_h[kHkv];
  a.tq = plan_h[kTotalQTiles];
  a.tk = plan_h[kTotalKTiles];
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const unsigned grid = (unsigned)plan_h[kNumItems];
  if (plan_h[kHeadDim] == 64)
    hipLaunchKernelGGL((prefill_kernel<64, true>), dim3(grid), dim3(kThreads), Tile<64>::kLds3, st, a);
  else
    hipLaunchKernelGGL((prefill_kernel<128, true>), dim3(grid), dim3(kThreads), Tile<128>::kLds3, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "prefill3 launch");
  return TILEMIX_OK;
}

int tilemix_quantize_k_fp8(const int32_t* plan_h, const int32_t* plan_d, const void* k_f16, uint8_t* k_f8,
                           float* k_scale_f8, void* hip_stream) {
  clear_error();
  int rc = check_plans(plan_h, plan_d);
  if (rc) return rc;
  const bool any = plan_h[kTotalTokens] > 0;
  if ((rc = check_dev_ptr(plan_d, "plan_d", true)) || (rc = check_dev_ptr(k_f16, "k_f16", any)) ||
      (rc = check_dev_ptr(k_f8, "k_f8", any)) || (rc = check_dev_ptr(k_scale_f8, "k_scale_f8", any)))
    return rc;
  if (!any) return TILEMIX_OK;
  QuantFp8Args a;
  a.plan = plan_d;
  a.q = nullptr;  // key blocks only
  a.k = static_cast<const _Float16*>(k_f16);
  a.qf8 = nullptr;
  a.kf8 = k_f8;
  a.qs = nullptr;
  a.ks = k_scale_f8;
  a.hq = plan_h[kHq];
  a.hkv = plan_h[kHkv];
  a.batch = plan_h[kBatch];
  a.tq = plan_h[kTotalQTiles];
  a.tk = plan_h[kTotalKTiles];
  const int64_t blocks = (int64_t)a.tk * a.hkv;
  if (blocks > 0x7fffffff) return fail(TILEMIX_EINVAL, "batch too large for one launch");
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (plan_h[kHeadDim] == 64)
    hipLaunchKernelGGL(quantize_qk_fp8_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(quantize_qk_fp8_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "quantize_k_fp8 launch");
  return TILEMIX_OK;
}

int tilemix_quantize_k_i8_fp8(const int32_t* plan_h, const int32_t* plan_d, const void* k_f16, int8_t* k_i8,
                              float* k_scale, uint8_t* k_f8, float* k_scale_f8, void* hip_stream) {
  clear_error();
  int rc = check_plans(plan_h, plan_d);
  if (rc) return rc;
  const bool any = plan_h[kTotalTokens] > 0;
  if ((rc = check_dev_ptr(plan_d, "plan_d", true)) || (rc = check_dev_ptr(k_f16, "k_f16", any)) ||
      (rc = check_dev_ptr(k_i8, "k_i8", any)) || (rc = check_dev_ptr(k_scale, "k_scale", any)) ||
      (rc = check_dev_ptr(k_f8, "k_f8", any)) || (rc = check_dev_ptr(k_scale_f8, "k_scale_f8", any)))
    return rc;
  if (!any) return TILEMIX_OK;
  QuantKBothArgs a;
  a.plan = plan_d;
  a.k = static_cast<const _Float16*>(k_f16);
  a.ki8 = k_i8;
  a.kf8 = k_f8;
  a.ks = k_scale;
  a.ksf8 = k_scale_f8;
  a.hkv = plan_h[kHkv];
  a.batch = plan_h[kBatch];
  a.tk = plan_h[kTotalKTiles];
  const int64_t blocks = (int64_t)a.tk * a.hkv;
  if (blocks > 0x7fffffff) return fail(TILEMIX_EINVAL, "batch too large for one launch");
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (plan_h[kHeadDim] == 64)
    hipLaunchKernelGGL(quantize_k_i8_fp8_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(quantize_k_i8_fp8_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "quantize_k_i8_fp8 launch");
  return TILEMIX_OK;
}

int tilemix_prefill_varlen3_qinline(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                                    const void* k_f16, const void* v_f16, const int8_t* k_i8,
                                    const float* k_scale, const uint8_t* k_f8, const float* k_scale_f8,
                                    const uint64_t* words_i8_d, const uint64_t* words_f8_d, void* out_f16,
                                    void* hip_stream) {
  clear_error();
  int rc = check_plans(plan_h, plan_d);
  if (rc) return rc;
  const bool any = plan_h[kNumItems] > 0;
  if ((rc = check_dev_ptr(plan_d, "plan_d", true)) || (rc = check_dev_ptr(q_f16, "q_f16", any)) ||
      (rc = check_dev_ptr(k_f16, "k_f16", any)) || (rc = check_dev_ptr(v_f16, "v_f16", any)) ||
      (rc = check_dev_ptr(k_i8, "k_i8", any)) || (rc = check_dev_ptr(k_scale, "k_scale", any)) ||
      (rc = check_dev_ptr(k_f8, "k_f8", any)) || (rc = check_dev_ptr(k_scale_f8, "k_scale_f8", any)) ||
      (rc = check_dev_ptr(words_i8_d, "words_i8_d", any)) || (rc = check_dev_ptr(words_f8_d, "words_f8_d", any)) ||
      (rc = check_dev_ptr(out_f16, "out_f16", any)))
    return rc;
  if (!any) return TILEMIX_OK;
  PrefillArgs a;
  a.plan = plan_d;
  a.q = static_cast<const _Float16*>(q_f16);
  a.k = static_cast<const _Float16*>(k_f16);
  a.v = static_cast<const _Float16*>(v_f16);
  a.qi8 = nullptr;  // Q is quantised in the kernel
  a.ki8 = k_i8;
  a.qs = nullptr;
  a.ks = k_scale;
  a.words = words_i8_d;
  a.out = static_cast<_Float16*>(out_f16);
  a.qf8 = nullptr;
  a.kf8 = k_f8;
  a.qsf8 = nullptr;
  a.ksf8 = k_scale_f8;
  a.wordsf8 = words_f8_d;
  a.hq = plan_h[kHq];
  a.hkv = plan_h[kHkv];
  a.tq = plan_h[kTotalQTiles];
  a.tk = plan_h[kTotalKTiles];
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const unsigned grid = (unsigned)plan_h[kNumItems];
  if (plan_h[kHeadDim] == 64)
    hipLaunchKernelGGL((prefill_kernel<64, true, true>), dim3(grid), dim3(kThreads), Tile<64>::kLds3Q, st, a);
  else
    hipLaunchKernelGGL((prefill_kernel<128, true, true>), dim3(grid), dim3(kThreads), Tile<128>::kLds3Q, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "prefill3_qinline launch");
  return TILEMIX_OK;
}

int tilemix_debug_qk_i32_tile(const int32_t* plan_h, const int32_t* plan_d, const int8_t* q_i8,
                              const int8_t* k_i8, int32_t seq, int32_t head, int32_t r, int32_t t,
                              int32_t* acc_d, void* hip_stream) {
  clear_error();
  int rc = check_plans(plan_h, plan_d);
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

int tilemix_debug_qk_f8_tile(const int32_t* plan_h, const int32_t* plan_d, const uint8_t* q_f8,
                             const uint8_t* k_f8, int32_t seq, int32_t head, int32_t r, int32_t t,
                             float* acc_d, void* hip_stream) {
  clear_error();
  int rc = check_plans(plan_h, plan_d);
  if (rc) return rc;
  if ((rc = check_dev_ptr(q_f8, "q_f8", true)) || (rc = check_dev_ptr(k_f8, "k_f8", true)) ||
      (rc = check_dev_ptr(acc_d, "acc_d", true)))
    return rc;
  if (seq < 0 || seq >= plan_h[kBatch]) return fail(TILEMIX_EINVAL, "seq %d out of range", seq);
  if (head < 0 || head >= plan_h[kHq]) return fail(TILEMIX_EINVAL, "head %d out of range", head);
  const int32_t* rec = plan_h + kHeaderLen + seq * kSeqStride;
  if (r < 0 || r >= rec[kSeqTm]) return fail(TILEMIX_EINVAL, "row %d out of range", r);
  if (t < 0 || t >= rec[kSeqTn]) return fail(TILEMIX_EINVAL, "key tile %d out of range", t);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (plan_h[kHeadDim] == 64)
    hipLaunchKernelGGL(debug_qk_f8_kernel<64>, dim3(1), dim3(kThreads), 0, st, plan_d, q_f8, k_f8, seq, head, r,
                       t, acc_d);
  else
    hipLaunchKernelGGL(debug_qk_f8_kernel<128>, dim3(1), dim3(kThreads), 0, st, plan_d, q_f8, k_f8, seq, head,
                       r, t, acc_d);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "debug fp8 tile launch");
  return TILEMIX_OK;
}

}  // extern "C"
