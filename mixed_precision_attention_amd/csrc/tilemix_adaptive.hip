// Per-group importance for adaptive routing words (gfx950).
//
// [Digest, setup]: the evaluated routing is static and data-free, and the
// interface accepts adaptive policies; [Map, "Placement can matter more
// than the nominal percentage"]: where reduced precision lands matters more
// than how much of it there is.  This is a cheap content statistic built
// from what the quantiser already produced:
//   * column sums of each int8 block's codes (Q: 128-row blocks per query
//     head, K: 64-row tiles per KV head);
//   * pooled score z(h, r, t) = fl32(dot) * fl32(fl32(s_q * s_k) / (n_q n_k)),
//     dot the exact integer dot product of the two column-sum vectors, n_q,
//     n_k the rows of the blocks (mean query against mean key);
//   * Z(kv, r, t) = max over the KV head's query heads;
//   * importance of group (r, G) = max of Z over its legal tiles minus the max
//     of Z over the row's legal tiles (binary32).
// The groups of each (sequence, KV head), ranked by (importance, r, G), route
// their first N8 to INT8: on the device (tilemix_select_routing_adaptive,
// below) or on the host (tilemix_build_routing_adaptive), bit-identical.  All
// arithmetic is exact or a fixed sequence of IEEE binary32 operations, so the
// result is reproducible bit for bit.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "tilemix.h"
#include "tilemix_host.h"
#include "tilemix_internal.h"

namespace tilemix {
namespace adaptive {

typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kMaxRowTiles = 4096;  // key tiles of one row held in LDS

struct ImpArgs {
  const int32_t* plan;
  const int8_t* qi8;
  const int8_t* ki8;
  const float* qs;
  const float* ks;
  int32_t* qsum;  // [Hq][tq][D]
  int32_t* ksum;  // [Hkv][tk][D]
  float* imp;     // [Hkv][tq][64]
  int32_t hq, hkv, batch, tq, tk;
};

__device__ inline int seq_of_tile(const int32_t* seqtab, int batch, int field, int tile) {
  int lo = 0, hi = batch - 1;  // last sequence whose first tile is <= tile
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seqtab[mid * kSeqStride + field] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Column sums of one (block, head): thread (16 columns, row part), 16-byte
// loads.
template <int D>
__global__ __launch_bounds__(kThreads) void block_colsum_kernel(ImpArgs a) {
  constexpr int kGroups = D / 16, kParts = kThreads / kGroups;
  __shared__ int part[kParts][D];
  const int32_t* seqtab = a.plan + kHeaderLen;
  int bid = blockIdx.x;
  const bool is_k = bid >= a.tq * a.hq;
  if (is_k) bid -= a.tq * a.hq;
  const int H = is_k ? a.hkv : a.hq, blk = is_k ? kBlockN : kBlockM;
  const int tile = bid / H, head = bid % H;
  const int s = seq_of_tile(seqtab, a.batch, is_k ? kSeqKtOff : kSeqQtOff, tile);
  const int32_t* rec = seqtab + s * kSeqStride;
  const int local = tile - rec[is_k ? kSeqKtOff : kSeqQtOff];
  const int row0 = rec[kSeqStart] + local * blk;
  const int nrows = min(blk, rec[kSeqLen] - local * blk);
  const int8_t* src = (is_k ? a.ki8 : a.qi8) + ((size_t)row0 * H + head) * D;
  const int tid = threadIdx.x, c16 = tid % kGroups, p = tid / kGroups;
  int acc[16] = {};
  for (int r = p; r < nrows; r += kParts) {
    const int4v w = *reinterpret_cast<const int4v*>(src + (size_t)r * H * D + c16 * 16);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] += (int)(int8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xff);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) part[p][c16 * 16 + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    int sum = 0;
#pragma unroll
    for (int q = 0; q < kParts; ++q) sum += part[q][tid];
    int32_t* dst = is_k ? a.ksum + ((size_t)head * a.tk + tile) * D : a.qsum + ((size_t)head * a.tq + tile) * D;
    dst[tid] = sum;
  }
}

// Importance of every group of one (KV head, query-tile row).  One thread
// per (key tile, query head): the column-sum dot product in float64, exact
// here (integer products below 2^27, sums below 2^35), so (float)dot is the
// binary32 rounding of the exact integer.
template <int D>
__global__ __launch_bounds__(kThreads) void importance_kernel(ImpArgs a) {
  __shared__ float zt[kMaxRowTiles];
  __shared__ float red[kThreads / 64];
  extern __shared__ double qsum_l[];  // [grp][D]
  const int32_t* seqtab = a.plan + kHeaderLen;
  const int kv = blockIdx.x / a.tq, tile = blockIdx.x % a.tq;
  const int s = seq_of_tile(seqtab, a.batch, kSeqQtOff, tile);
  const int32_t* rec = seqtab + s * kSeqStride;
  const int r = tile - rec[kSeqQtOff], L = rec[kSeqLen], g = rec[kSeqG], kt0 = rec[kSeqKtOff];
  const int nt = min(kBlockM * r + kBlockM - 1, L - 1) / kBlockN + 1;
  const int grp = a.hq / a.hkv, h0 = kv * grp;
  const int nq = min(kBlockM, L - kBlockM * r);
  const int tid = threadIdx.x;
  for (int i = tid; i < grp * D; i += kThreads)
    qsum_l[i] = (double)a.qsum[((size_t)(h0 + i / D) * a.tq + tile) * D + i % D];
  for (int t = tid; t < nt; t += kThreads) zt[t] = -INFINITY;
  __syncthreads();
  // Z(t) = max over the query heads of fl32(dot) * fl32(fl32(s_q s_k) / (n_q n_k))
  for (int item = tid; item < nt * grp; item += kThreads) {
    const int t = item / grp, h = item % grp;
    const int kt = kt0 + t;
    const int nk = min(kBlockN, L - kBlockN * t);
    const int4v* ksr = reinterpret_cast<const int4v*>(a.ksum + ((size_t)kv * a.tk + kt) * D);
    const double* qh = qsum_l + h * D;
    // four independent exact partial sums (every partial sum is an integer
    // well inside float64's exact range, so the order does not matter)
    double d4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
    for (int c4 = 0; c4 < D / 4; ++c4) {
      const int4v kk = ksr[c4];
#pragma unroll
      for (int e = 0; e < 4; ++e) d4[e] = __builtin_fma(qh[4 * c4 + e], (double)kk[e], d4[e]);
    }
    const double dot = (d4[0] + d4[1]) + (d4[2] + d4[3]);
    const float sk = a.ks[(size_t)kv * a.tk + kt];
    const float aa = __fmul_rn(a.qs[(size_t)(h0 + h) * a.tq + tile], sk);
    const float b = __fdiv_rn(aa, (float)(nq * nk));
    // the max over heads is order-independent: combine them in LDS (each
    // failed exchange means another head raised the slot, so at most grp
    // rounds)
    const float z = __fmul_rn((float)dot, b);
    float* slot = &zt[t];
    float old = *slot;
    while (z > old) {
      const unsigned prev = atomicCAS(reinterpret_cast<unsigned*>(slot), __float_as_uint(old), __float_as_uint(z));
      if (prev == __float_as_uint(old)) break;
      old = __uint_as_float(prev);
    }
  }
  __syncthreads();
  float rowmax = -INFINITY;
  for (int t = tid; t < nt; t += kThreads) rowmax = fmaxf(rowmax, zt[t]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) rowmax = fmaxf(rowmax, __shfl_xor(rowmax, off));
  if ((tid & 63) == 0) red[tid >> 6] = rowmax;
  __syncthreads();
  rowmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int ngroups = (nt - 1) / g + 1;
  if (tid < kWordBits) {
    float v = INFINITY;  // illegal groups
    if (tid < ngroups) {
      float zg = -INFINITY;
      for (int t = tid * g; t < min(tid * g + g, nt); ++t) zg = fmaxf(zg, zt[t]);
      v = __fsub_rn(zg, rowmax);
    }
    a.imp[((size_t)kv * a.tq + tile) * kWordBits + tid] = v;
  }
}

}  // namespace adaptive
}  // namespace tilemix

using namespace tilemix;
using namespace tilemix::adaptive;

namespace {

int check_ptr(const void* p, const char* name, bool needed) {
  if (!needed) return TILEMIX_OK;
  if (p == nullptr) return fail(TILEMIX_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(TILEMIX_EINVAL, "%s is not 16-byte aligned", name);
  return TILEMIX_OK;
}

// --------------------------------------------------------------------------
// Selection of the adaptive words on the device: one workgroup of 1,024
// threads per (sequence, KV head) routes the N8 least important legal
// groups to INT8 under the total order (importance, r, G), the order of the
// host ranking (tilemix_build_routing_adaptive), so the words are the same
// bit for bit:
//   * key: the importance as an order-preserving unsigned integer (-0 mapped
//     to +0 so that equal values tie as a floating-point comparison has
//     them; NaN after +inf);
//   * a four-pass radix select, 8 bits a pass from the top, finds the N8-th
//     smallest key T (an LDS histogram of the candidates' next digit per
//     pass, one wave scanning it);
//   * a group is INT8 when its key is below T, or equal to T and among the
//     first of the equal keys in (r, G) order, as many as N8 still needs;
//   * the importance layout's slots [row][64] are visited 1,024 at a time in
//     (r, G) order, so each wave holds one row's 64 groups: the equal keys'
//     running count is a ballot popcount plus the earlier waves' and rounds'
//     counts, and the row's word is a ballot.
// --------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

struct SelArgs {
  const int32_t* plan;
  const float* imp;  // [Hkv][tq][64]
  uint64_t* words;   // [Hkv][tq]
  int32_t hkv, tq, coverage_bp;
};

__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  const uint32_t mag = u & 0x7fffffffu;
  if (mag == 0) return 0x80000000u;              // -0 and +0 alike
  if (mag > 0x7f800000u) return 0xffffffffu;     // NaN after +inf
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline int last_group_of(int r, int L, int g) {
  const int last_q = min(r * kBlockM + kBlockM - 1, L - 1);
  return (last_q / kBlockN) / g;
}

__global__ __launch_bounds__(kSelThreads) void select_words_kernel(SelArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_cnt[kSelWaves];
  __shared__ uint32_t s_bin, s_below_bin, s_nlegal;
  const int seq = blockIdx.x / a.hkv, kv = blockIdx.x % a.hkv;
  const int32_t* rec = a.plan + kHeaderLen + seq * kSeqStride;
  const int L = rec[kSeqLen], g = rec[kSeqG], Tm = rec[kSeqTm], qt = rec[kSeqQtOff];
  if (Tm == 0) return;  // the whole workgroup, before any barrier
  const float* imp = a.imp + ((size_t)kv * a.tq + qt) * kWordBits;
  uint64_t* words = a.words + (size_t)kv * a.tq + qt;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rounds = (Tm + kSelWaves - 1) / kSelWaves;  // a wave per row each round

  // legal groups of the sequence and the INT8 count
  if (tid == 0) s_nlegal = 0;
  __syncthreads();
  {
    uint32_t n = 0;
    for (int r = tid; r < Tm; r += kSelThreads) n += (uint32_t)last_group_of(r, L, g) + 1;
    if (n) atomicAdd(&s_nlegal, n);
  }
  __syncthreads();
  const int64_t n_legal = s_nlegal;
  const int64_t n8 = ((int64_t)a.coverage_bp * n_legal + 5000) / 10000;
  if (n8 == 0) {
    for (int r = tid; r < Tm; r += kSelThreads) words[r] = 0ull;
    return;
  }

  // radix select of the n8-th smallest key
  uint32_t prefix = 0, mask = 0;
  int64_t rank = n8 - 1;  // index of the wanted key among the candidates
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int k = 0; k < rounds; ++k) {
      const int r = k * kSelWaves + w;
      if (r < Tm && lane <= last_group_of(r, L, g)) {
        const uint32_t key = order_key(imp[(size_t)r * kWordBits + lane]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    if (w == 0) {
      // lane l holds bins 4l .. 4l + 3; exclusive scan over the lanes
      uint32_t c[4], tot = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = hist[4 * lane + i];
        tot += c[i];
      }
      uint32_t incl = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      uint32_t before = incl - tot;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if ((int64_t)before <= rank && rank < (int64_t)before + c[i]) {
          s_bin = 4 * lane + i;
          s_below_bin = before;
        }
        before += c[i];
      }
    }
    __syncthreads();
    prefix |= s_bin << shift;
    mask |= 255u << shift;
    rank -= s_below_bin;
    __syncthreads();  // s_bin is rewritten by the next pass
  }
  const uint32_t T = prefix;
  const int64_t need_eq = rank + 1;  // equal keys still routed, in (r, G) order

  // words: one row per wave per round
  int64_t carry = 0;
  for (int k = 0; k < rounds; ++k) {
    const int r = k * kSelWaves + w;
    const bool valid = r < Tm && lane <= last_group_of(r, L, g);
    const uint32_t key = valid ? order_key(imp[(size_t)r * kWordBits + lane]) : 0u;
    const bool lt = valid && key < T, eq = valid && key == T;
    const uint64_t be = __ballot(eq);
    if (lane == 0) wave_cnt[w] = (uint32_t)__popcll(be);
    __syncthreads();
    uint32_t wave_off = 0, round_tot = 0;
#pragma unroll
    for (int u = 0; u < kSelWaves; ++u) {
      const uint32_t cu = wave_cnt[u];
      if (u < w) wave_off += cu;
      round_tot += cu;
    }
    const int64_t eq_idx = carry + wave_off + __popcll(be & ((1ull << lane) - 1ull));
    const bool int8 = lt || (eq && eq_idx < need_eq);
    const uint64_t word = __ballot(int8);
    if (lane == 0 && r < Tm) words[r] = word;
    carry += round_tot;
    __syncthreads();  // wave_cnt is rewritten next round
  }
}

}  // namespace

extern "C" {

int tilemix_importance_workspace_size(const int32_t* plan_h, int64_t* bytes) {
  clear_error();
  int rc = check_plan(plan_h);
  if (rc) return rc;
  if (bytes == nullptr) return fail(TILEMIX_EINVAL, "bytes is NULL");
  *bytes = ((int64_t)plan_h[kHq] * plan_h[kTotalQTiles] + (int64_t)plan_h[kHkv] * plan_h[kTotalKTiles]) *
           plan_h[kHeadDim] * (int64_t)sizeof(int32_t);
  return TILEMIX_OK;
}

int tilemix_routing_importance(const int32_t* plan_h, const int32_t* plan_d, const int8_t* q_i8,
                               const int8_t* k_i8, const float* q_scale, const float* k_scale,
                               void* workspace, int64_t workspace_bytes, float* importance_d,
                               void* hip_stream) {
  clear_error();
  int rc = check_plans(plan_h, plan_d);
  if (rc) return rc;
  const bool any = plan_h[kTotalTokens] > 0;
  if ((rc = check_ptr(plan_d, "plan_d", true)) || (rc = check_ptr(q_i8, "q_i8", any)) ||
      (rc = check_ptr(k_i8, "k_i8", any)) || (rc = check_ptr(q_scale, "q_scale", any)) ||
      (rc = check_ptr(k_scale, "k_scale", any)) || (rc = check_ptr(workspace, "workspace", any)) ||
      (rc = check_ptr(importance_d, "importance_d", any)))
    return rc;
  int64_t need = 0;
  tilemix_importance_workspace_size(plan_h, &need);
  if (workspace_bytes < need)
    return fail(TILEMIX_EINVAL, "workspace holds %lld bytes, needs %lld", (long long)workspace_bytes,
                (long long)need);
  for (int32_t s = 0; s < plan_h[kBatch]; ++s)
    if (plan_h[kHeaderLen + s * kSeqStride + kSeqTn] > kMaxRowTiles)
      return fail(TILEMIX_EUNSUPPORTED, "sequence %d is longer than %d tokens", s, kMaxRowTiles * kBlockN);
  if (!any) return TILEMIX_OK;
  ImpArgs a;
  a.plan = plan_d;
  a.qi8 = q_i8;
  a.ki8 = k_i8;
  a.qs = q_scale;
  a.ks = k_scale;
  a.hq = plan_h[kHq];
  a.hkv = plan_h[kHkv];
  a.batch = plan_h[kBatch];
  a.tq = plan_h[kTotalQTiles];
  a.tk = plan_h[kTotalKTiles];
  a.qsum = static_cast<int32_t*>(workspace);
  a.ksum = a.qsum + (size_t)a.hq * a.tq * plan_h[kHeadDim];
  a.imp = importance_d;
  const int d = plan_h[kHeadDim];
  const int64_t b1 = (int64_t)a.tq * a.hq + (int64_t)a.tk * a.hkv, b2 = (int64_t)a.hkv * a.tq;
  if (b1 > 0x7fffffff || b2 > 0x7fffffff) return fail(TILEMIX_EINVAL, "batch too large for one launch");
  const size_t lds = (size_t)(a.hq / a.hkv) * d * sizeof(double);
  if (lds > 64 * 1024) return fail(TILEMIX_EUNSUPPORTED, "too many query heads per KV head");
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (d == 64) {
    hipLaunchKernelGGL(block_colsum_kernel<64>, dim3((unsigned)b1), dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL(importance_kernel<64>, dim3((unsigned)b2), dim3(kThreads), lds, st, a);
  } else {
    hipLaunchKernelGGL(block_colsum_kernel<128>, dim3((unsigned)b1), dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL(importance_kernel<128>, dim3((unsigned)b2), dim3(kThreads), lds, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TILEMIX_EHIP, "importance launch: %s", hipGetErrorString(e));
  return TILEMIX_OK;
}

int tilemix_select_routing_adaptive(const int32_t* plan_h, const int32_t* plan_d, const float* importance_d,
                                    int32_t coverage_bp, uint64_t* words_d, int64_t* int8_groups_h,
                                    int64_t* legal_groups_h, void* hip_stream) {
  clear_error();
  int rc = check_plans(plan_h, plan_d);
  if (rc) return rc;
  if (coverage_bp < 0 || coverage_bp > 10000)
    return fail(TILEMIX_EINVAL, "coverage_bp must be in [0, 10000] (got %d)", coverage_bp);
  const int32_t batch = plan_h[kBatch], hkv = plan_h[kHkv];
  // the counts, from the plan's geometry (the kernel derives the same)
  for (int32_t s = 0; s < batch; ++s) {
    const int32_t* rec = plan_h + kHeaderLen + s * kSeqStride;
    const int64_t L = rec[kSeqLen], g = rec[kSeqG], Tm = rec[kSeqTm];
    int64_t n = 0;
    for (int64_t r = 0; r < Tm; ++r) n += (std::min(r * kBlockM + kBlockM - 1, L - 1) / kBlockN) / g + 1;
    if (legal_groups_h) legal_groups_h[s] = n;
    if (int8_groups_h) int8_groups_h[s] = (coverage_bp * n + 5000) / 10000;
  }
  const bool any = plan_h[kTotalQTiles] > 0;
  if ((rc = check_ptr(plan_d, "plan_d", true)) || (rc = check_ptr(importance_d, "importance_d", any)) ||
      (rc = check_ptr(words_d, "words_d", any)))
    return rc;
  if (!any) return TILEMIX_OK;
  const int64_t blocks = (int64_t)batch * hkv;
  if (blocks > 0x7fffffff) return fail(TILEMIX_EINVAL, "batch too large for one launch");
  SelArgs a;
  a.plan = plan_d;
  a.imp = importance_d;
  a.words = words_d;
  a.hkv = hkv;
  a.tq = plan_h[kTotalQTiles];
  a.coverage_bp = coverage_bp;
  hipLaunchKernelGGL(select_words_kernel, dim3((unsigned)blocks), dim3(kSelThreads), 0,
                     static_cast<hipStream_t>(hip_stream), a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TILEMIX_EHIP, "word selection launch: %s", hipGetErrorString(e));
  return TILEMIX_OK;
}

}  // extern "C"
