// TileMix decode step against an INT8 key/value cache (gfx950).
//
// [Explainer, 支持的场景]; [Digest, setup]: TileMix also serves the decode
// side with an INT8 key/value cache.  One decode step: every sequence has one
// new query, the token at position L - 1 whose key and value are already in
// the cache; it attends to all L cached positions.  Key tile t is routed by
// bit t / g of the prefill word of the query-tile row holding L - 1 ([Map,
// hot loop]):
//   bit 1: INT8 query (one scale per sequence and head) . INT8 key, int32
//          accumulation, times s_q * s_k / sqrt(d) ([Digest, method]);
//   bit 0: FP16 query . dequantised key (k_i8 * s_k), times 1 / sqrt(d).
// P is rounded to fp16 and multiplies the dequantised value v_i8 * s_v.
//
// The step reads the whole cache once and does a few operations per byte, so
// it is bound by HBM bandwidth: plain vector-ALU dot products, no matrix
// instructions.  Split over the keys (256 per workgroup) so that even a small
// batch fills the chip; a second kernel merges the partial softmax states.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "tilemix.h"
#include "tilemix_host.h"
#include "tilemix_internal.h"

namespace tilemix {
namespace decode {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;            // 4 waves of 64
constexpr int kChunk = 4 * kBlockN;      // keys per workgroup: one key tile per wave
constexpr int kMaxG = 8;                 // query heads per workgroup
constexpr float kLog2e = 1.44269504088896340736f;

// --------------------------------------------------------------------------
// Cache quantiser: K and V in the prefill quantiser's key blocks (64 x d per
// head, scale = absmax / 127, q = round-half-even(x / s) clamped to +-127,
// IEEE binary32 division).  One workgroup per (block, head, operand).
// --------------------------------------------------------------------------
struct KvQuantArgs {
  const int32_t* plan;
  const _Float16* k;
  const _Float16* v;
  int8_t* ki8;
  int8_t* vi8;
  float* ks;
  float* vs;
  int32_t hkv, batch, tk;
};

__device__ inline int seq_of_key_tile(const int32_t* seqtab, int batch, int tile) {
  int lo = 0, hi = batch - 1;  // last sequence whose first key tile is <= tile
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seqtab[mid * kSeqStride + kSeqKtOff] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int D>
__global__ __launch_bounds__(kThreads) void quantize_kv_kernel(KvQuantArgs a) {
  constexpr int kChunksPerRow = D / 8;  // 16-byte chunks of one row
  constexpr int kPerThread = kBlockN * kChunksPerRow / kThreads;
  __shared__ float red[4];
  const int32_t* seqtab = a.plan + kHeaderLen;
  int bid = blockIdx.x;
  const bool is_v = bid >= a.tk * a.hkv;
  if (is_v) bid -= a.tk * a.hkv;
  const int tile = bid / a.hkv, head = bid % a.hkv;
  const int s = seq_of_key_tile(seqtab, a.batch, tile);
  const int32_t* rec = seqtab + s * kSeqStride;
  const int local = tile - rec[kSeqKtOff];
  const int row0 = rec[kSeqStart] + local * kBlockN;
  const int nrows = min(kBlockN, rec[kSeqLen] - local * kBlockN);
  const size_t base = ((size_t)row0 * a.hkv + head) * D;
  const _Float16* src = (is_v ? a.v : a.k) + base;
  int8_t* dst = (is_v ? a.vi8 : a.ki8) + base;
  const int stride = a.hkv * D;

  const int tid = threadIdx.x;
  half8 vals[kPerThread];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int idx = tid + i * kThreads;
    const int r = idx / kChunksPerRow, cc = idx % kChunksPerRow;
    half8 x = {};
    if (r < nrows) x = *reinterpret_cast<const half8*>(src + (size_t)r * stride + cc * 8);
    vals[i] = x;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((float)x[j]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = __fdiv_rn(amax, 127.0f);
  if (tid == 0) (is_v ? a.vs : a.ks)[(size_t)head * a.tk + tile] = sc;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int idx = tid + i * kThreads;
    const int r = idx / kChunksPerRow, cc = idx % kChunksPerRow;
    if (r >= nrows) continue;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float qf = amax > 0.f ? __builtin_rintf(__fdiv_rn((float)vals[i][j], sc)) : 0.f;
      const uint32_t b = (uint32_t)((int)__builtin_amdgcn_fmed3f(qf, -127.f, 127.f) & 0xff);
      if (j < 4) lo |= b << (8 * j); else hi |= b << (8 * (j - 4));
    }
    *reinterpret_cast<uint2*>(dst + (size_t)r * stride + cc * 8) = make_uint2(lo, hi);
  }
}

// --------------------------------------------------------------------------
// Partial step: one workgroup per (256-key chunk, sequence, KV head, group of
// up to 8 query heads).  Wave w scores key tile 4 c + w, one key per lane;
// the chunk's softmax state (m, l, unnormalised O) goes to the workspace.
// --------------------------------------------------------------------------
struct DecodeArgs {
  const int32_t* plan;
  const _Float16* q;     // [B, Hq, D]
  const int8_t* ki8;     // [T, Hkv, D]
  const int8_t* vi8;     // [T, Hkv, D]
  const float* ks;       // [Hkv, tk]
  const float* vs;       // [Hkv, tk]
  const uint64_t* words; // [Hkv, tq]
  float* work;           // [B, Hq, chunks, D + 2]
  _Float16* out;         // [B, Hq, D]
  int32_t batch, hq, hkv, tq, tk, chunks, head_groups;
};

template <int D>
struct Smem {
  _Float16 qf[kMaxG][D];                            // fp16 queries
  int8_t qi[kMaxG][D];                              // int8 queries
  float sq[kMaxG];                                  // query scales
  float mx[4][kMaxG];                               // per-wave maxima
  float ls[4][kMaxG];                               // per-wave sums of P
  _Float16 pv[kMaxG][kChunk];                       // fp16-rounded P
  float part[4][kMaxG][D];                          // per-wave P.V sums
};

// Signed int8 x4 -> two fp16 pairs, exactly: bytes b + 128 become the low
// mantissa byte of 1024 + (b + 128) and the bias 1152 is subtracted.
__device__ inline void i8x4_to_half(uint32_t w, half2v& lo, half2v& hi) {
  const uint32_t x = w ^ 0x80808080u;
  const half2v bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u)) - bias;
  hi = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u)) - bias;
}

// kG: query heads of the workgroup known at compile time when a KV head has
// fewer than kMaxG of them (kG = kMaxG: a runtime count, the last group of a
// larger set may be partial).
template <int D, int kG>
__global__ __launch_bounds__(kThreads, 4) void decode_partial_kernel(DecodeArgs a) {
  __shared__ Smem<D> sm;
  const int chunk = blockIdx.x;
  const int hg = blockIdx.y % a.head_groups;
  const int sk = blockIdx.y / a.head_groups;  // sequence * Hkv + kv
  const int seq = sk / a.hkv, kv = sk % a.hkv;
  const int32_t* rec = a.plan + kHeaderLen + seq * kSeqStride;
  const int start = rec[kSeqStart], L = rec[kSeqLen];
  if (chunk * kChunk >= L) return;  // no keys here (the merge reads only live chunks)
  const int grp = a.hq / a.hkv;
  const int h0 = kv * grp + hg * kMaxG;
  const int G = kG < kMaxG ? kG : min(kMaxG, grp - hg * kMaxG);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float inv_sqrt_d = (float)(1.0 / std::sqrt((double)D));

  // Every load of the workgroup is issued up front -- the queries first, then
  // this lane's key row and this thread's share of the staged values -- so
  // their latencies overlap.
  const int t = chunk * 4 + w;              // this wave's key tile (sequence-local)
  const int j = t * kBlockN + lane;         // this lane's key
  const bool live = j < L;
  const bool tile_live = t * kBlockN < L;
  _Float16 qv[2][D / 64];                   // heads w and w + 4 of the group
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int i = 0; i < D / 64; ++i)
      qv[u][i] = w + 4 * u < G ? a.q[((size_t)seq * a.hq + h0 + w + 4 * u) * D + lane + 64 * i]
                               : (_Float16)0.0f;
  uint32_t kw[D / 4] = {};
  if (live) {
    const int4v* krow = reinterpret_cast<const int4v*>(a.ki8 + ((size_t)(start + j) * a.hkv + kv) * D);
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const int4v x = krow[i];
      kw[4 * i] = x[0]; kw[4 * i + 1] = x[1]; kw[4 * i + 2] = x[2]; kw[4 * i + 3] = x[3];
    }
  }
  // Values in the P.V layout: thread (4 channels c4, key part) holds its 4
  // channels of each of its keys (a wave reads whole 128-byte rows).
  constexpr int kGroups = D / 4, kParts = kThreads / kGroups, kKeys = kChunk / kParts;
  const int c4 = tid % kGroups, part = tid / kGroups;
  uint32_t vreg[kKeys];
#pragma unroll
  for (int k = 0; k < kKeys; ++k) {
    const int jj = chunk * kChunk + part * kKeys + k;
    vreg[k] = jj < L ? *reinterpret_cast<const uint32_t*>(a.vi8 + ((size_t)(start + jj) * a.hkv + kv) * D + c4 * 4)
                     : 0u;
  }
  const int vt = chunk * 4 + part * kKeys / kBlockN;  // key tile of this part
  const float s_vp = vt * kBlockN < L ? a.vs[(size_t)kv * a.tk + rec[kSeqKtOff] + vt] : 0.f;
  const int kt = rec[kSeqKtOff] + t;
  const float s_k = tile_live ? a.ks[(size_t)kv * a.tk + kt] : 0.f;
  const uint64_t word = a.words[(size_t)kv * a.tq + rec[kSeqQtOff] + (L - 1) / kBlockM];
  const bool bit = tile_live && ((word >> (t / rec[kSeqG])) & 1ull);

  // Queries of the group: fp16 copy, and the int8 copy with one scale per
  // (sequence, head) -- the quantiser with a block of one row.
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int h = w + 4 * u;
    if (h >= G) break;
    float x[D / 64];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      sm.qf[h][lane + 64 * i] = qv[u][i];
      x[i] = (float)qv[u][i];
      amax = fmaxf(amax, fabsf(x[i]));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float sq = __fdiv_rn(amax, 127.0f);
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      const float qq = amax > 0.f ? __builtin_rintf(__fdiv_rn(x[i], sq)) : 0.f;
      sm.qi[h][lane + 64 * i] = (int8_t)(int)__builtin_amdgcn_fmed3f(qq, -127.f, 127.f);
    }
    if (lane == 0) sm.sq[h] = sq;
  }
  __syncthreads();

  // Scores of this wave's key tile, one key per lane, in the log2 domain.
  float xs[kG];
  if (bit) {
#pragma unroll
    for (int h = 0; h < kG; ++h) {
      if (h >= G) break;
      const uint32_t* qw = reinterpret_cast<const uint32_t*>(sm.qi[h]);
      int acc = 0;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) acc = __builtin_amdgcn_sdot4((int)qw[i], (int)kw[i], acc, false);
      // exact: |acc| <= 127^2 d < 2^24
      const float f = (sm.sq[h] * s_k) * inv_sqrt_d;
      xs[h] = (float)acc * f * kLog2e;
    }
  } else {
    half2v kh[D / 2];
#pragma unroll
    for (int i = 0; i < D / 4; ++i) i8x4_to_half(kw[i], kh[2 * i], kh[2 * i + 1]);
    const float f = s_k * inv_sqrt_d * kLog2e;
#pragma unroll
    for (int h = 0; h < kG; ++h) {
      if (h >= G) break;
      const half2v* qh = reinterpret_cast<const half2v*>(sm.qf[h]);
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < D / 2; ++i) acc = __builtin_amdgcn_fdot2(qh[i], kh[i], acc, false);
      xs[h] = acc * f;
    }
  }

  // Chunk softmax state per head (log2 domain, relative to the chunk max).
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    if (h >= G) break;
    float m = live ? xs[h] : -INFINITY;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) sm.mx[w][h] = m;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    if (h >= G) break;
    const float m = fmaxf(fmaxf(sm.mx[0][h], sm.mx[1][h]), fmaxf(sm.mx[2][h], sm.mx[3][h]));
    // P rounded to fp16; the normaliser sums the same rounded values
    const float p = live ? (float)(_Float16)__builtin_amdgcn_exp2f(xs[h] - m) : 0.f;
    sm.pv[h][w * kBlockN + lane] = (_Float16)p;
    float l = p;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0) sm.ls[w][h] = l;
  }
  __syncthreads();

  // P.V with the dequantised values: each thread sums its keys two at a time
  // with fp16 pair dot products (fp16 P and int8 values are exact in fp16;
  // products exact, fp32 sums), then applies its key tile's value scale (a
  // part lies inside one key tile).
  float acc[kG][4] = {};
#pragma unroll
  for (int k = 0; k < kKeys; k += 2) {
    const int key = part * kKeys + k;
    // (channel c of key, of key + 1) pairs for the 4 channels
    half2v v01[4];
    i8x4_to_half(__builtin_amdgcn_perm(vreg[k + 1], vreg[k], 0x05010400u), v01[0], v01[1]);
    i8x4_to_half(__builtin_amdgcn_perm(vreg[k + 1], vreg[k], 0x07030602u), v01[2], v01[3]);
#pragma unroll
    for (int h = 0; h < kG; ++h) {
      if (h >= G) break;
      const half2v pp = *reinterpret_cast<const half2v*>(&sm.pv[h][key]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[h][e] = __builtin_amdgcn_fdot2(pp, v01[e], acc[h][e], false);
    }
  }
  // Sum the parts: lanes l, l + kGroups, ... of a wave hold the same
  // channels, then the four waves through LDS.
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    if (h >= G) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = acc[h][e] * s_vp;
#pragma unroll
      for (int off = kGroups; off < 64; off <<= 1) x += __shfl_xor(x, off);
      if (lane < kGroups) sm.part[w][h][c4 * 4 + e] = x;
    }
  }
  __syncthreads();
  // Workspace record of (sequence, head, chunk): m, l, O[D] (unnormalised).
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D, c = idx % D;
    float o = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) o += sm.part[p][h][c];
    float* rec_out = a.work + (((size_t)seq * a.hq + h0 + h) * a.chunks + chunk) * (D + 2);
    rec_out[2 + c] = o;
    if (c == 0) {
      rec_out[0] = fmaxf(fmaxf(sm.mx[0][h], sm.mx[1][h]), fmaxf(sm.mx[2][h], sm.mx[3][h]));
      rec_out[1] = (sm.ls[0][h] + sm.ls[1][h]) + (sm.ls[2][h] + sm.ls[3][h]);
    }
  }
}

// Merge of the chunks of one (sequence, query head), one wave each: the
// online-softmax combination of partial states ([Routes, precision routing]:
// one shared state), O = sum 2^(m_i - M) O_i / sum 2^(m_i - M) l_i, written
// as fp16.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(DecodeArgs a) {
  const int wid = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wid >= a.batch * a.hq) return;
  const int seq = wid / a.hq, h = wid % a.hq;
  const int L = a.plan[kHeaderLen + seq * kSeqStride + kSeqLen];
  _Float16* o = a.out + ((size_t)seq * a.hq + h) * D;
  if (L == 0) {
#pragma unroll
    for (int i = 0; i < D / 64; ++i) o[lane + 64 * i] = (_Float16)0.0f;
    return;
  }
  const int n = (L + kChunk - 1) / kChunk;
  const float* base = a.work + ((size_t)seq * a.hq + h) * a.chunks * (D + 2);
  float M = -INFINITY;
  for (int i = lane; i < n; i += 64) M = fmaxf(M, base[(size_t)i * (D + 2)]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float l = 0.f;
  for (int i = lane; i < n; i += 64) {
    const float* r = base + (size_t)i * (D + 2);
    l += __builtin_amdgcn_exp2f(r[0] - M) * r[1];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
  float acc[D / 64] = {};
#pragma unroll 16
  for (int i = 0; i < n; ++i) {
    const float* r = base + (size_t)i * (D + 2);
    const float wgt = __builtin_amdgcn_exp2f(r[0] - M);
#pragma unroll
    for (int c = 0; c < D / 64; ++c) acc[c] += wgt * r[2 + lane + 64 * c];
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int c = 0; c < D / 64; ++c) o[lane + 64 * c] = (_Float16)(acc[c] * inv);
}

}  // namespace decode
}  // namespace tilemix

using namespace tilemix;
using namespace tilemix::decode;

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

template <int D>
void launch_partial(int kg, dim3 grid, hipStream_t st, const DecodeArgs& a) {
  switch (kg) {
    case 1: hipLaunchKernelGGL((decode_partial_kernel<D, 1>), grid, dim3(kThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((decode_partial_kernel<D, 2>), grid, dim3(kThreads), 0, st, a); break;
    case 3: hipLaunchKernelGGL((decode_partial_kernel<D, 3>), grid, dim3(kThreads), 0, st, a); break;
    case 4: hipLaunchKernelGGL((decode_partial_kernel<D, 4>), grid, dim3(kThreads), 0, st, a); break;
    case 5: hipLaunchKernelGGL((decode_partial_kernel<D, 5>), grid, dim3(kThreads), 0, st, a); break;
    case 6: hipLaunchKernelGGL((decode_partial_kernel<D, 6>), grid, dim3(kThreads), 0, st, a); break;
    case 7: hipLaunchKernelGGL((decode_partial_kernel<D, 7>), grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((decode_partial_kernel<D, kMaxG>), grid, dim3(kThreads), 0, st, a); break;
  }
}

// Chunks of the longest sequence.
int64_t max_chunks(const int32_t* plan_h) {
  int64_t m = 0;
  for (int32_t s = 0; s < plan_h[kBatch]; ++s) {
    const int64_t L = plan_h[kHeaderLen + s * kSeqStride + kSeqLen];
    m = std::max(m, (L + kChunk - 1) / kChunk);
  }
  return m;
}

}  // namespace

extern "C" {

int tilemix_quantize_kv(const int32_t* plan_h, const int32_t* plan_d, const void* k_f16,
                        const void* v_f16, int8_t* k_i8, int8_t* v_i8, float* k_scale,
                        float* v_scale, void* hip_stream) {
  clear_error();
  int rc = check_plan(plan_h);
  if (rc) return rc;
  const bool any = plan_h[kTotalTokens] > 0;
  if ((rc = check_ptr(plan_d, "plan_d", true)) || (rc = check_ptr(k_f16, "k_f16", any)) ||
      (rc = check_ptr(v_f16, "v_f16", any)) || (rc = check_ptr(k_i8, "k_i8", any)) ||
      (rc = check_ptr(v_i8, "v_i8", any)) || (rc = check_ptr(k_scale, "k_scale", any)) ||
      (rc = check_ptr(v_scale, "v_scale", any)))
    return rc;
  if (!any) return TILEMIX_OK;
  KvQuantArgs a;
  a.plan = plan_d;
  a.k = static_cast<const _Float16*>(k_f16);
  a.v = static_cast<const _Float16*>(v_f16);
  a.ki8 = k_i8;
  a.vi8 = v_i8;
  a.ks = k_scale;
  a.vs = v_scale;
  a.hkv = plan_h[kHkv];
  a.batch = plan_h[kBatch];
  a.tk = plan_h[kTotalKTiles];
  const int64_t blocks = 2 * (int64_t)a.tk * a.hkv;
  if (blocks > 0x7fffffff) return fail(TILEMIX_EINVAL, "cache too large for one launch");
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (plan_h[kHeadDim] == 64)
    hipLaunchKernelGGL(quantize_kv_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(quantize_kv_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "cache quantize launch");
  return TILEMIX_OK;
}

int tilemix_decode_workspace_size(const int32_t* plan_h, int64_t* bytes) {
  clear_error();
  int rc = check_plan(plan_h);
  if (rc) return rc;
  if (bytes == nullptr) return fail(TILEMIX_EINVAL, "bytes is NULL");
  *bytes = (int64_t)plan_h[kBatch] * plan_h[kHq] * max_chunks(plan_h) * (plan_h[kHeadDim] + 2) *
           (int64_t)sizeof(float);
  return TILEMIX_OK;
}

int tilemix_decode_varlen(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                          const int8_t* k_i8, const int8_t* v_i8, const float* k_scale,
                          const float* v_scale, const uint64_t* words_d, void* workspace,
                          int64_t workspace_bytes, void* out_f16, void* hip_stream) {
  clear_error();
  int rc = check_plan(plan_h);
  if (rc) return rc;
  const int32_t batch = plan_h[kBatch];
  const bool any = plan_h[kTotalTokens] > 0;
  if ((rc = check_ptr(plan_d, "plan_d", true)) || (rc = check_ptr(q_f16, "q_f16", batch > 0)) ||
      (rc = check_ptr(k_i8, "k_i8", any)) || (rc = check_ptr(v_i8, "v_i8", any)) ||
      (rc = check_ptr(k_scale, "k_scale", any)) || (rc = check_ptr(v_scale, "v_scale", any)) ||
      (rc = check_ptr(words_d, "words_d", any)) || (rc = check_ptr(workspace, "workspace", any)) ||
      (rc = check_ptr(out_f16, "out_f16", batch > 0)))
    return rc;
  int64_t need = 0;
  tilemix_decode_workspace_size(plan_h, &need);
  if (workspace_bytes < need)
    return fail(TILEMIX_EINVAL, "workspace holds %lld bytes, needs %lld", (long long)workspace_bytes,
                (long long)need);
  if (batch == 0) return TILEMIX_OK;
  DecodeArgs a;
  a.plan = plan_d;
  a.q = static_cast<const _Float16*>(q_f16);
  a.ki8 = k_i8;
  a.vi8 = v_i8;
  a.ks = k_scale;
  a.vs = v_scale;
  a.words = words_d;
  a.work = static_cast<float*>(workspace);
  a.out = static_cast<_Float16*>(out_f16);
  a.batch = batch;
  a.hq = plan_h[kHq];
  a.hkv = plan_h[kHkv];
  a.tq = plan_h[kTotalQTiles];
  a.tk = plan_h[kTotalKTiles];
  a.chunks = (int32_t)max_chunks(plan_h);
  const int grp = a.hq / a.hkv;
  a.head_groups = (grp + kMaxG - 1) / kMaxG;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const int64_t gy = (int64_t)batch * a.hkv * a.head_groups;
  if (gy > 65535 || a.chunks > 0x7fffffff) return fail(TILEMIX_EINVAL, "batch too large for one launch");
  const int d = plan_h[kHeadDim];
  if (a.chunks > 0) {
    const dim3 grid(a.chunks, (unsigned)gy);
    const int kg = std::min(grp, kMaxG);
    if (d == 64) launch_partial<64>(kg, grid, st, a);
    else launch_partial<128>(kg, grid, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "decode launch");
  }
  const unsigned merge = (unsigned)(((int64_t)batch * a.hq + 3) / 4);  // one wave per (sequence, head)
  if (d == 64)
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(merge), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(merge), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "decode merge launch");
  return TILEMIX_OK;
}

}  // extern "C"
