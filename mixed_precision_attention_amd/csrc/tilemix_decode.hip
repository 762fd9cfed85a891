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
#include <mutex>

#include "tilemix.h"
#include "tilemix_host.h"
#include "tilemix_internal.h"

// Scratch of the allocation-free decode entry point: the partial-softmax
// records, in a static device array (one copy per GPU the library runs on,
// held until the process ends).  Host code never passes the array's name to a
// kernel: its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[TILEMIX_DECODE_SCRATCH_BYTES];

namespace tilemix {
namespace decode {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;            // 4 waves of 64
constexpr int kChunk = 4 * kBlockN;      // keys per workgroup: one key tile per wave
// Query heads per workgroup: larger GQA groups split into groups of 4 (the
// last may be smaller), whose workgroups read the same cache rows (the
// second read mostly from cache): four heads fit four workgroups per CU,
// where eight took 190 registers and two per CU (28/4-head varlen step
// 51.3 -> 49.4 us, the output bit-identical).
constexpr int kMaxG = 4;
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
// Partial step: one workgroup per (KV head and group of up to 4 query heads,
// 256-key chunk, sequence), the KV head fastest in the launch order so that
// workgroups running side by side read neighbouring bytes of the same cache
// rows.  Wave w scores key tile 4 c + w; the chunk's softmax state (m, l,
// unnormalised O) goes to the workspace.
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
  float mx[4][kMaxG];                               // per-wave (key tile) maxima
  float ls[4][kMaxG];                               // per-wave sums of P
  _Float16 pv[kMaxG][kChunk];                       // fp16-rounded P
  float part[4][kMaxG][D];                          // per-wave P.V sums
};

// Lane exchanges within groups of 8 (or 4) lanes for the score reduction:
// the partner's bit b of the lane index is the opposite of this lane's.
template <int kMask>
__device__ inline int xchg(int x) {
  if constexpr (kMask == 1) return __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  else if constexpr (kMask == 2) return __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  else return __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);  // row_half_mirror: lane ^ 7
}
template <int kMask>
__device__ inline float xchg(float x) { return __builtin_bit_cast(float, xchg<kMask>(__builtin_bit_cast(int, x))); }

// Sums n = kLanes partial values across the kLanes lanes that share a key
// row and leaves lane (index mod kLanes = i) with the full sum of value i:
// at each step a lane keeps the half of its values that its bit selects and
// adds the partner's copy of that half (recursive halving).
template <int kLanes, typename T>
__device__ inline T transpose_reduce(T (&v)[kLanes], int lane) {
  if constexpr (kLanes == 8) {
    const bool b = lane & 4;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const T send = b ? v[k] : v[k + 4];
      v[k] = (b ? v[k + 4] : v[k]) + xchg<4>(send);
    }
  }
  {
    const bool b = lane & 2;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const T send = b ? v[k] : v[k + 2];
      v[k] = (b ? v[k + 2] : v[k]) + xchg<2>(send);
    }
  }
  const bool b = lane & 1;
  const T send = b ? v[0] : v[1];
  return (b ? v[1] : v[0]) + xchg<1>(send);
}

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
  const int kv = blockIdx.x / a.head_groups, hg = blockIdx.x % a.head_groups;
  const int chunk = blockIdx.y, seq = blockIdx.z;
  const int32_t* rec = a.plan + kHeaderLen + seq * kSeqStride;
  const int start = rec[kSeqStart], L = rec[kSeqLen];
  if (chunk * kChunk >= L) return;  // no keys here (the merge folds in only live chunks)
  const int grp = a.hq / a.hkv;
  const int h0 = kv * grp + hg * kMaxG;
  const int G = kG < kMaxG ? kG : min(kMaxG, grp - hg * kMaxG);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float inv_sqrt_d = (float)(1.0 / std::sqrt((double)D));

  // Every load of the workgroup is issued up front, branch-free (the scale
  // and query indices clamped into range, the key and value rows through the
  // buffer resources below), in the order of first use -- the scalars, the
  // queries, the wave's key tile, then this thread's share of the values --
  // so the waits before the scores and before P.V each cover only what they
  // need, and the values stream in while the scores are computed.
  //
  // Key tile layout: kLanes = d / 16 lanes share a key row, each holding 16
  // bytes (channels 16 sub ..) of rows kRows i + r, i < kLanes, so that one
  // load instruction covers whole 128-byte lines (one row per lane asks the
  // memory pipeline for 64 lines per instruction and streams a third slower).
  // After the cross-lane reduction lane (r, sub) holds the score of key
  // kRows sub + r of the tile.
  constexpr int kLanes = D / 16, kRows = 64 / kLanes;
  const int r = lane / kLanes, sub = lane % kLanes;
  const int t = chunk * 4 + w;                        // this wave's key tile (sequence-local)
  const int kk = w * kBlockN + sub * kRows + r;       // this lane's key within the chunk
  const bool live = chunk * kChunk + kk < L;
  const bool tile_live = t * kBlockN < L;
  constexpr int kGroups = D / 4, kParts = kThreads / kGroups, kKeys = kChunk / kParts;
  const int c4 = tid % kGroups, part = tid / kGroups;
  const int vt = chunk * 4 + part * kKeys / kBlockN;  // key tile of this part
  const int kt_off = rec[kSeqKtOff];
  const float s_vp_raw = a.vs[(size_t)kv * a.tk + kt_off + min(vt, (L - 1) / kBlockN)];
  const float s_k_raw = a.ks[(size_t)kv * a.tk + kt_off + min(t, (L - 1) / kBlockN)];
  const uint64_t word = a.words[(size_t)kv * a.tq + rec[kSeqQtOff] + (L - 1) / kBlockM];
  constexpr int kQPerWave = (kMaxG + 3) / 4;  // query heads each wave quantises
  _Float16 qv[kQPerWave][D / 64];             // heads w, w + 4, ... of the group
#pragma unroll
  for (int u = 0; u < kQPerWave; ++u)
#pragma unroll
    for (int i = 0; i < D / 64; ++i)
      qv[u][i] = a.q[((size_t)seq * a.hq + h0 + min(w + 4 * u, G - 1)) * D + lane + 64 * i];
  // The chunk's rows of this head through buffer resources sized to the rows
  // before the sequence end: a row at or past it lies outside and reads as
  // zero (its score is masked and its P is 0), and each load's address is
  // one lane offset (the range check covers the lane offset, so the row
  // step goes there, not in the scalar offset).
  const uint32_t stride = (uint32_t)(a.hkv * D);      // bytes between consecutive rows
  const int nrows = min(kChunk, L - chunk * kChunk);  // >= 1
  const size_t row0 = ((size_t)(start + chunk * kChunk) * a.hkv + kv) * D;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.ki8 + row0), (short)0, (int)(nrows * stride), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.vi8 + row0), (short)0, (int)(nrows * stride), 0x00020000);
  int4v kx[kLanes];
  const uint32_t koff = (uint32_t)(w * kBlockN + r) * stride + sub * 16;
#pragma unroll
  for (int i = 0; i < kLanes; ++i) kx[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, koff + kRows * i * stride, 0, 0);
  __builtin_amdgcn_sched_barrier(0);  // keep the key loads ahead of the value loads
  // Values in the P.V layout: thread (4 channels c4, key part) holds its 4
  // channels of each of its keys (a wave reads whole 128-byte rows).
  uint32_t vreg[kKeys];
  const uint32_t voff = (uint32_t)(part * kKeys) * stride + c4 * 4;
#pragma unroll
  for (int k = 0; k < kKeys; ++k) vreg[k] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(vrs, voff + k * stride, 0, 0);
  const float s_vp = vt * kBlockN < L ? s_vp_raw : 0.f;
  const float s_k = tile_live ? s_k_raw : 0.f;
  const bool bit = tile_live && ((word >> (t / rec[kSeqG])) & 1ull);

  // Queries of the group: fp16 copy, and the int8 copy with one scale per
  // (sequence, head) -- the quantiser with a block of one row.
#pragma unroll
  for (int u = 0; u < kQPerWave; ++u) {
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

  // Scores of this wave's key tile in the log2 domain: each lane's 16
  // channels of its kLanes rows, then summed across the row's lanes.
  float xs[kG];
  if (bit) {
#pragma unroll
    for (int h = 0; h < kG; ++h) {
      if (h >= G) break;
      const int4v qq = *reinterpret_cast<const int4v*>(&sm.qi[h][sub * 16]);
      int pr[kLanes];
#pragma unroll
      for (int i = 0; i < kLanes; ++i) {
        int acc = __builtin_amdgcn_sdot4(qq[0], kx[i][0], 0, false);
        acc = __builtin_amdgcn_sdot4(qq[1], kx[i][1], acc, false);
        acc = __builtin_amdgcn_sdot4(qq[2], kx[i][2], acc, false);
        pr[i] = __builtin_amdgcn_sdot4(qq[3], kx[i][3], acc, false);
      }
      // exact: |sum| <= 127^2 d < 2^24
      const int acc = transpose_reduce<kLanes>(pr, lane);
      const float f = (sm.sq[h] * s_k) * inv_sqrt_d;
      xs[h] = (float)acc * f * kLog2e;
    }
  } else {
    half2v kh[kLanes][8];
#pragma unroll
    for (int i = 0; i < kLanes; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) i8x4_to_half((uint32_t)kx[i][e], kh[i][2 * e], kh[i][2 * e + 1]);
    const float f = s_k * inv_sqrt_d * kLog2e;
#pragma unroll
    for (int h = 0; h < kG; ++h) {
      if (h >= G) break;
      const half8 q0 = *reinterpret_cast<const half8*>(&sm.qf[h][sub * 16]);
      const half8 q1 = *reinterpret_cast<const half8*>(&sm.qf[h][sub * 16 + 8]);
      const half2v qh[8] = {q0.s01, q0.s23, q0.s45, q0.s67, q1.s01, q1.s23, q1.s45, q1.s67};
      float pr[kLanes];
#pragma unroll
      for (int i = 0; i < kLanes; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_fdot2(qh[e], kh[i][e], acc, false);
        pr[i] = acc;
      }
      xs[h] = transpose_reduce<kLanes>(pr, lane) * f;
    }
  }

  // Softmax state per wave and head over the wave's own key tile (log2
  // domain, relative to the tile's maximum): P is rounded to fp16 against it
  // and the normaliser sums the same rounded values.  The wave reads back
  // only the P it wrote, so no workgroup barrier stands between a wave's
  // keys and its P.V; the four tiles' states are combined at the end,
  // rescaled to the chunk maximum (the online-softmax step with the key tile
  // as the unit).
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    if (h >= G) break;
    float m = live ? xs[h] : -INFINITY;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float p = live ? (float)(_Float16)__builtin_amdgcn_exp2f(xs[h] - m) : 0.f;
    sm.pv[h][kk] = (_Float16)p;
    float l = p;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0) {  // read only after the final barrier
      sm.mx[w][h] = m;
      sm.ls[w][h] = l;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // P.V with the dequantised values over the wave's own 64 keys: each thread
  // sums its keys two at a time with fp16 pair dot products (fp16 P and int8
  // values are exact in fp16; products exact, fp32 sums), then applies its
  // key tile's value scale (a part lies inside one key tile).
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
  // channels; then the four waves' states through LDS.
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
  // Workspace record of (sequence, head, chunk): m, l, O[D] (unnormalised),
  // O = sum over the tiles of 2^(m_w - m) O_w.
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D, c = idx % D;
    const float m = fmaxf(fmaxf(sm.mx[0][h], sm.mx[1][h]), fmaxf(sm.mx[2][h], sm.mx[3][h]));
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float mp = sm.mx[p][h];
      const float sc = mp == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mp - m);
      o += sc * sm.part[p][h][c];
      l += sc * sm.ls[p][h];
    }
    float* rec_out = a.work + (((size_t)seq * a.hq + h0 + h) * a.chunks + chunk) * (D + 2);
    rec_out[2 + c] = o;
    if (c == 0) {
      rec_out[0] = m;
      rec_out[1] = l;
    }
  }
}

// Merge of the chunks of one (sequence, query head), one workgroup of
// kMergeWaves(n) waves each: the online-softmax combination of partial
// states ([Routes, precision routing]: one shared state),
// O = sum 2^(m_i - M) O_i / sum 2^(m_i - M) l_i, written as fp16.
constexpr int kMergeBatch = 16;     // chunk records a wave requests together
constexpr int kMergeMaxWaves = 8;

// Waves per merge workgroup for a longest sequence of `chunks` chunks: one
// batch of 16 chunk records per wave, up to 8 waves.
inline int merge_waves(int64_t chunks) {
  const int64_t b = (chunks + kMergeBatch - 1) / kMergeBatch;
  return (int)std::max<int64_t>(1, std::min<int64_t>(kMergeMaxWaves, b));
}

template <int D>
__global__ __launch_bounds__(64 * kMergeMaxWaves) void decode_merge_kernel(DecodeArgs a) {
  __shared__ float sm_m[kMergeMaxWaves], sm_l[kMergeMaxWaves];
  __shared__ float sm_o[kMergeMaxWaves][D];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int seq = blockIdx.x / a.hq, h = blockIdx.x % a.hq;
  const float* base = a.work + ((size_t)seq * a.hq + h) * a.chunks * (D + 2);
  // The sequence's length and the wave's first batch of records are
  // requested together: the batch covers the chunks any sequence of the
  // launch can have (all of them written or not), and the length decides
  // afterwards which of them are live, so the merge waits one memory latency
  // before folding.  Wave w takes batches w, w + nw, ...; a batch's (m, l)
  // and O rows are requested together and the next batch before this one is
  // folded in (online-softmax rescale across batches).
  const int L = a.plan[kHeaderLen + seq * kSeqStride + kSeqLen];
  float2 ml, mln;
  float ov[kMergeBatch][D / 64], ovn[kMergeBatch][D / 64];
  auto fetch = [&](int i0, float2& m2, float (&dst)[kMergeBatch][D / 64]) {
    const int nb = min(kMergeBatch, a.chunks - i0);  // records inside the workspace
    m2 = lane < nb ? *reinterpret_cast<const float2*>(base + (size_t)(i0 + lane) * (D + 2))
                   : make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i)
#pragma unroll
      for (int c = 0; c < D / 64; ++c)
        dst[i][c] = i < nb ? base[(size_t)(i0 + i) * (D + 2) + 2 + lane + 64 * c] : 0.f;
  };
  const int step = nw * kMergeBatch;
  int i0 = w * kMergeBatch;
  if (i0 < a.chunks) fetch(i0, mln, ovn);
  const int n = (L + kChunk - 1) / kChunk;  // live chunks of this sequence
  float M = -INFINITY, l = 0.f;
  float acc[D / 64] = {};
  for (; i0 < n; i0 += step) {
    ml = mln;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i)
#pragma unroll
      for (int c = 0; c < D / 64; ++c) ov[i][c] = ovn[i][c];
    if (i0 + step < n) fetch(i0 + step, mln, ovn);
    const int nb = min(kMergeBatch, n - i0);
    if (lane >= nb) ml = make_float2(-INFINITY, 0.f);  // records past the sequence's end
    float mb = ml.x;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mb = fmaxf(mb, __shfl_xor(mb, off));
    const float Mn = fmaxf(M, mb);
    const float alpha = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
    const float wl = lane < nb ? __builtin_amdgcn_exp2f(ml.x - Mn) : 0.f;
    float lb = wl * ml.y;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lb += __shfl_xor(lb, off);
    l = l * alpha + lb;
#pragma unroll
    for (int c = 0; c < D / 64; ++c) acc[c] *= alpha;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const float wi = __shfl(wl, i);
      if (i < nb) {
#pragma unroll
        for (int c = 0; c < D / 64; ++c) acc[c] += wi * ov[i][c];
      }
    }
    M = Mn;
  }
  if (nw > 1) {  // combine the waves' states
    if (lane == 0) { sm_m[w] = M; sm_l[w] = l; }
#pragma unroll
    for (int c = 0; c < D / 64; ++c) sm_o[w][lane + 64 * c] = acc[c];
    __syncthreads();
    if (w != 0) return;
    float Mt = -INFINITY;
    for (int u = 0; u < nw; ++u) Mt = fmaxf(Mt, sm_m[u]);
    l = 0.f;
#pragma unroll
    for (int c = 0; c < D / 64; ++c) acc[c] = 0.f;
    for (int u = 0; u < nw; ++u) {
      const float wu = sm_m[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm_m[u] - Mt);
      l += wu * sm_l[u];
#pragma unroll
      for (int c = 0; c < D / 64; ++c) acc[c] += wu * sm_o[u][lane + 64 * c];
    }
  }
  _Float16* o = a.out + ((size_t)seq * a.hq + h) * D;
  const float inv = l > 0.f ? 1.0f / l : 0.f;  // an empty sequence gives zeros
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

constexpr int64_t kDecodeScratchBytes = TILEMIX_DECODE_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int decode_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(TILEMIX_EUNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(TILEMIX_EHIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TILEMIX_OK;
}

// The decode step's launches, with the partial records at `work`
// (the caller checked its size).
int decode_launch(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16, const int8_t* k_i8,
                  const int8_t* v_i8, const float* k_scale, const float* v_scale, const uint64_t* words_d,
                  float* work, void* out_f16, void* hip_stream) {
  const int32_t batch = plan_h[kBatch];
  if (batch == 0) return TILEMIX_OK;
  DecodeArgs a;
  a.plan = plan_d;
  a.q = static_cast<const _Float16*>(q_f16);
  a.ki8 = k_i8;
  a.vi8 = v_i8;
  a.ks = k_scale;
  a.vs = v_scale;
  a.words = words_d;
  a.work = work;
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
  if (batch > 65535) return fail(TILEMIX_EINVAL, "batch of %d sequences too large for one launch", batch);
  if ((int64_t)a.hkv * plan_h[kHeadDim] * kChunk > 0x7fffffff)
    return fail(TILEMIX_EINVAL, "%d KV heads: a 256-row chunk of the cache exceeds 2 GiB", a.hkv);
  if (a.chunks > 65535)
    return fail(TILEMIX_EINVAL, "a sequence of more than %d keys is too long for one launch", 65535 * kChunk);
  const int d = plan_h[kHeadDim];
  if (a.chunks > 0) {
    const dim3 grid((unsigned)(a.hkv * a.head_groups), (unsigned)a.chunks, (unsigned)batch);
    const int kg = std::min(grp, kMaxG);
    if (d == 64) launch_partial<64>(kg, grid, st, a);
    else launch_partial<128>(kg, grid, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "decode launch");
  }
  const unsigned merge = (unsigned)((int64_t)batch * a.hq);  // one workgroup per (sequence, head)
  const dim3 mblock(64 * merge_waves(a.chunks));
  if (d == 64)
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(merge), mblock, 0, st, a);
  else
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(merge), mblock, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "decode merge launch");
  return TILEMIX_OK;
}

int decode_check(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16, const int8_t* k_i8,
                 const int8_t* v_i8, const float* k_scale, const float* v_scale, const uint64_t* words_d,
                 void* out_f16) {
  int rc = check_plans(plan_h, plan_d);
  if (rc) return rc;
  const int32_t batch = plan_h[kBatch];
  const bool any = plan_h[kTotalTokens] > 0;
  if ((rc = check_ptr(plan_d, "plan_d", true)) || (rc = check_ptr(q_f16, "q_f16", batch > 0)) ||
      (rc = check_ptr(k_i8, "k_i8", any)) || (rc = check_ptr(v_i8, "v_i8", any)) ||
      (rc = check_ptr(k_scale, "k_scale", any)) || (rc = check_ptr(v_scale, "v_scale", any)) ||
      (rc = check_ptr(words_d, "words_d", any)) || (rc = check_ptr(out_f16, "out_f16", batch > 0)))
    return rc;
  return TILEMIX_OK;
}

}  // namespace

extern "C" {

int tilemix_quantize_kv(const int32_t* plan_h, const int32_t* plan_d, const void* k_f16,
                        const void* v_f16, int8_t* k_i8, int8_t* v_i8, float* k_scale,
                        float* v_scale, void* hip_stream) {
  clear_error();
  int rc = check_plans(plan_h, plan_d);
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
  int rc = decode_check(plan_h, plan_d, q_f16, k_i8, v_i8, k_scale, v_scale, words_d, out_f16);
  if (rc) return rc;
  if ((rc = check_ptr(workspace, "workspace", plan_h[kTotalTokens] > 0))) return rc;
  int64_t need = 0;
  tilemix_decode_workspace_size(plan_h, &need);
  if (workspace_bytes < need)
    return fail(TILEMIX_EINVAL, "workspace holds %lld bytes, needs %lld", (long long)workspace_bytes,
                (long long)need);
  return decode_launch(plan_h, plan_d, q_f16, k_i8, v_i8, k_scale, v_scale, words_d,
                       static_cast<float*>(workspace), out_f16, hip_stream);
}

int tilemix_decode_varlen_noalloc(const int32_t* plan_h, const int32_t* plan_d, const void* q_f16,
                                  const int8_t* k_i8, const int8_t* v_i8, const float* k_scale,
                                  const float* v_scale, const uint64_t* words_d, void* out_f16,
                                  void* hip_stream) {
  clear_error();
  int rc = decode_check(plan_h, plan_d, q_f16, k_i8, v_i8, k_scale, v_scale, words_d, out_f16);
  if (rc) return rc;
  int64_t need = 0;
  tilemix_decode_workspace_size(plan_h, &need);
  if (need > kDecodeScratchBytes)
    return fail(TILEMIX_EINVAL, "decode step needs %lld bytes of scratch, more than the %lld the "
                "allocation-free entry point holds; use tilemix_decode_varlen with a workspace",
                (long long)need, (long long)kDecodeScratchBytes);
  void* work = nullptr;
  if ((rc = decode_scratch(&work))) return rc;
  return decode_launch(plan_h, plan_d, q_f16, k_i8, v_i8, k_scale, v_scale, words_d,
                       static_cast<float*>(work), out_f16, hip_stream);
}

}  // extern "C"
