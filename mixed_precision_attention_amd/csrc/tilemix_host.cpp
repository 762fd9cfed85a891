// Host half of libtilemix: argument validation, error reporting, the routing
// word builder and the work planner.  Plain C++ (no device code).
//
// Sources (web pages about TileMix), cited by title and section:
//   [Digest]    "TileMix: Tile-Centric Mixed-Precision Attention for LLM
//               Inference Acceleration" (paper digest), method and setup.
//   [Explainer] "TileMix：给AI大模型的“注意力”做一次精准的精度分配手术"
//               (popular explainer), sections 第二步 and 支持的场景.

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "tilemix.h"
#include "tilemix_internal.h"
#include "tilemix_host.h"

namespace tilemix {

namespace {
thread_local std::string g_last_error;
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

const char* last_error() { return g_last_error.c_str(); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_cu_seqlens(const int32_t* cu, int32_t batch) {
  if (batch < 0) return fail(TILEMIX_EINVAL, "batch must be >= 0 (got %d)", batch);
  if (cu == nullptr) return fail(TILEMIX_EINVAL, "cu_seqlens_h is NULL");
  if (cu[0] != 0) return fail(TILEMIX_EINVAL, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
  for (int32_t i = 0; i < batch; ++i)
    if (cu[i + 1] < cu[i])
      return fail(TILEMIX_EINVAL, "cu_seqlens must be non-decreasing (index %d)", i + 1);
  return TILEMIX_OK;
}

// ---------------------------------------------------------------------------
// Geometry.  [Digest, method]: BLOCK_M x BLOCK_N tiles; adjacent key tiles form
// one routing group per bit; g keeps the groups of a row within 64 bits.
// ---------------------------------------------------------------------------
SeqGeo geometry(int64_t L) {
  SeqGeo s;
  s.L = L;
  s.Tm = (L + kBlockM - 1) / kBlockM;
  s.Tn = (L + kBlockN - 1) / kBlockN;
  s.g = std::max<int64_t>(1, (s.Tn + kWordBits - 1) / kWordBits);
  return s;
}

int64_t SeqGeo::last_tile(int64_t r) const {
  const int64_t last_q = std::min<int64_t>(kBlockM * r + kBlockM - 1, L - 1);
  return last_q / kBlockN;
}

int64_t SeqGeo::last_group(int64_t r) const { return last_tile(r) / g; }

namespace {

// ---------------------------------------------------------------------------
// Routing templates.  Each template is a strict total order of the legal
// groups (r, G) of one sequence, FP16-first; the coverage keeps the first
// N_legal - N8 in FP16.  With d = D(r) - G and n_r = D(r) + 1:
//   Band (d, r, G); Global (G, r); Row-Random ((2 rho+1)/(2 n_r), r, G) with
//   rho the rank of G in its row by (hash, G); Aligned-Sparse
//   ((2d+1)/(2 n_r), r, G); SpTrans = round-robin union of the stride order
//   (d mod s != 0, d, r, G), s = max(1, isqrt(n of last row)), and Band;
//   BigBird = round-robin union of Band, Global and Row-Random.
// ---------------------------------------------------------------------------
struct Group {
  int32_t r, G;
};

// splitmix64 output finaliser (Steele, Lea and Flood 2014).
uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Row-Random hash of a group, keyed on the sequence-local row and group only,
// so one template serves every sequence and KV head.
uint64_t group_hash(uint64_t seed, int64_t r, int64_t G) {
  return mix64(mix64(seed) ^ static_cast<uint64_t>(kWordBits * r + G));
}

// a/b < c/d for positive denominators.
inline bool frac_less(int64_t a, int64_t b, int64_t c, int64_t d) { return a * d < c * b; }
inline bool frac_eq(int64_t a, int64_t b, int64_t c, int64_t d) { return a * d == c * b; }

std::vector<Group> legal_groups(const SeqGeo& geo) {
  std::vector<Group> v;
  for (int64_t r = 0; r < geo.Tm; ++r)
    for (int64_t G = 0; G <= geo.last_group(r); ++G) v.push_back({(int32_t)r, (int32_t)G});
  return v;
}

std::vector<Group> order_band(const SeqGeo& geo) {
  auto v = legal_groups(geo);
  std::sort(v.begin(), v.end(), [&](const Group& x, const Group& y) {
    const int64_t dx = geo.last_group(x.r) - x.G, dy = geo.last_group(y.r) - y.G;
    if (dx != dy) return dx < dy;
    if (x.r != y.r) return x.r < y.r;
    return x.G < y.G;
  });
  return v;
}

std::vector<Group> order_global(const SeqGeo& geo) {
  auto v = legal_groups(geo);
  std::sort(v.begin(), v.end(), [](const Group& x, const Group& y) {
    if (x.G != y.G) return x.G < y.G;
    return x.r < y.r;
  });
  return v;
}

// Sort by a fractional key num/den (den > 0), ties by (r, G).
template <typename NumDen>
std::vector<Group> order_by_fraction(const SeqGeo& geo, NumDen key) {
  auto v = legal_groups(geo);
  std::sort(v.begin(), v.end(), [&](const Group& x, const Group& y) {
    int64_t nx, dx, ny, dy;
    key(x, nx, dx);
    key(y, ny, dy);
    if (!frac_eq(nx, dx, ny, dy)) return frac_less(nx, dx, ny, dy);
    if (x.r != y.r) return x.r < y.r;
    return x.G < y.G;
  });
  return v;
}

std::vector<Group> order_rowrandom(const SeqGeo& geo, uint64_t seed) {
  // rank[r][G]: position of G in row r when sorted by (hash, G)
  std::vector<std::vector<int32_t>> rank(geo.Tm);
  for (int64_t r = 0; r < geo.Tm; ++r) {
    const int64_t n = geo.last_group(r) + 1;
    std::vector<std::pair<uint64_t, int32_t>> hs(n);
    for (int64_t G = 0; G < n; ++G) hs[G] = {group_hash(seed, r, G), (int32_t)G};
    std::sort(hs.begin(), hs.end());
    rank[r].assign(n, 0);
    for (int64_t i = 0; i < n; ++i) rank[r][hs[i].second] = (int32_t)i;
  }
  return order_by_fraction(geo, [&](const Group& x, int64_t& num, int64_t& den) {
    num = 2 * (int64_t)rank[x.r][x.G] + 1;
    den = 2 * (geo.last_group(x.r) + 1);
  });
}

std::vector<Group> order_alignedsparse(const SeqGeo& geo) {
  return order_by_fraction(geo, [&](const Group& x, int64_t& num, int64_t& den) {
    num = 2 * (geo.last_group(x.r) - x.G) + 1;
    den = 2 * (geo.last_group(x.r) + 1);
  });
}

int64_t isqrt64(int64_t n) {
  int64_t s = 0;
  while ((s + 1) * (s + 1) <= n) ++s;
  return s;
}

// Round-robin union: each order in turn contributes its next group not taken.
std::vector<Group> round_robin_union(const SeqGeo& geo, const std::vector<std::vector<Group>>& orders) {
  const size_t total = orders.empty() ? 0 : orders[0].size();
  // taken flag indexed by (row start offset + G)
  std::vector<int64_t> row_base(geo.Tm + 1, 0);
  for (int64_t r = 0; r < geo.Tm; ++r) row_base[r + 1] = row_base[r] + geo.last_group(r) + 1;
  std::vector<char> taken(row_base[geo.Tm], 0);
  std::vector<size_t> pos(orders.size(), 0);
  std::vector<Group> out;
  out.reserve(total);
  while (out.size() < total) {
    for (size_t i = 0; i < orders.size() && out.size() < total; ++i) {
      const auto& o = orders[i];
      while (pos[i] < o.size() && taken[row_base[o[pos[i]].r] + o[pos[i]].G]) ++pos[i];
      if (pos[i] < o.size()) {
        const Group x = o[pos[i]++];
        taken[row_base[x.r] + x.G] = 1;
        out.push_back(x);
      }
    }
  }
  return out;
}

std::vector<Group> order_sptrans(const SeqGeo& geo) {
  const int64_t s = geo.Tm ? std::max<int64_t>(1, isqrt64(geo.last_group(geo.Tm - 1) + 1)) : 1;
  auto stride = legal_groups(geo);
  std::sort(stride.begin(), stride.end(), [&](const Group& x, const Group& y) {
    const int64_t dx = geo.last_group(x.r) - x.G, dy = geo.last_group(y.r) - y.G;
    const int ox = (dx % s) != 0, oy = (dy % s) != 0;
    if (ox != oy) return ox < oy;
    if (dx != dy) return dx < dy;
    if (x.r != y.r) return x.r < y.r;
    return x.G < y.G;
  });
  return round_robin_union(geo, {stride, order_band(geo)});
}

std::vector<Group> template_order(const SeqGeo& geo, int32_t tmpl, uint64_t seed) {
  switch (tmpl) {
    case TILEMIX_BAND: return order_band(geo);
    case TILEMIX_GLOBAL: return order_global(geo);
    case TILEMIX_ROWRANDOM: return order_rowrandom(geo, seed);
    case TILEMIX_ALIGNEDSPARSE: return order_alignedsparse(geo);
    case TILEMIX_BIGBIRD:
      return round_robin_union(geo, {order_band(geo), order_global(geo), order_rowrandom(geo, seed)});
    case TILEMIX_SPTRANS: return order_sptrans(geo);
    default: return {};
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Planner
// ---------------------------------------------------------------------------
int64_t plan_length(const int32_t* plan_h) {
  return kHeaderLen + (int64_t)plan_h[kBatch] * kSeqStride + (int64_t)plan_h[kNumItems] * kItemStride;
}

uint32_t plan_hash(const int32_t* plan_h) {
  // Four interleaved FNV-1a streams over 32-bit words (word i feeds stream
  // i mod 4, the hash field counts as 0), folded together at the end: the
  // multiply chains are a quarter as long as one byte-wise stream, so a plan
  // of tens of kilobytes is checked in a few microseconds on every call.
  constexpr uint32_t kPrime = 16777619u;
  uint32_t h[4] = {2166136261u, 2166136261u ^ 1u, 2166136261u ^ 2u, 2166136261u ^ 3u};
  const int64_t n = plan_length(plan_h);
  int64_t i = 0;
  for (; i + 4 <= n; i += 4)
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = (i + j == kPlanHash) ? 0u : (uint32_t)plan_h[i + j];
      h[j] = (h[j] ^ w) * kPrime;
    }
  for (int j = 0; i < n; ++i, ++j) h[j] = (h[j] ^ (i == kPlanHash ? 0u : (uint32_t)plan_h[i])) * kPrime;
  uint32_t r = 2166136261u;
  for (int j = 0; j < 4; ++j)
    for (int b = 0; b < 4; ++b) r = (r ^ ((h[j] >> (8 * b)) & 0xffu)) * kPrime;
  return r ^ (uint32_t)n;
}

// The header's fields are checked for consistency before the hash reads the
// body, so a damaged header cannot send the check past the plan's end.
int check_plan(const int32_t* plan_h) {
  if (plan_h == nullptr) return fail(TILEMIX_EINVAL, "plan_h is NULL");
  if (plan_h[kMagic] != kPlanMagic) return fail(TILEMIX_EINVAL, "plan_h is not a TileMix plan");
  if (plan_h[kVersion] != kPlanVersion)
    return fail(TILEMIX_EUNSUPPORTED, "plan version %d, library expects %d", plan_h[kVersion],
                kPlanVersion);
  const int32_t batch = plan_h[kBatch];
  if (batch < 0 || plan_h[kHq] <= 0 || plan_h[kHkv] <= 0 || plan_h[kHq] % plan_h[kHkv] != 0 ||
      (plan_h[kHeadDim] != 64 && plan_h[kHeadDim] != 128) || plan_h[kNumItems] < 0 ||
      plan_h[kSeqOff] != kHeaderLen || plan_h[kItemOff] != kHeaderLen + batch * kSeqStride)
    return fail(TILEMIX_EINVAL, "plan_h header is inconsistent");
  if ((uint32_t)plan_h[kPlanHash] != plan_hash(plan_h))
    return fail(TILEMIX_EINVAL, "plan_h does not match its checksum (modified or truncated plan)");
  return TILEMIX_OK;
}

namespace {

struct Unit {
  int32_t seq, head, row;
  int64_t cost;  // key tiles the row visits
};

constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

// Build the launch-ordered unit list.  Units sharing a (sequence, KV head)
// stay on one die, so their K/V tiles are reused from that die's L2; a group
// whose work exceeds half a die's share is dealt into several parts.  Parts
// are assigned to dies by longest-processing-time; each die's queue runs its
// longest rows first.  The hardware hands workgroup b to die b mod 8, so the
// per-die queues are interleaved into the launch order.
std::vector<Unit> schedule(const std::vector<SeqGeo>& geos, int32_t hq, int32_t hkv) {
  const int32_t grp = hq / hkv;
  std::vector<std::vector<Unit>> parts;
  int64_t total = 0;
  std::vector<std::vector<Unit>> groups;
  for (size_t s = 0; s < geos.size(); ++s) {
    for (int32_t kv = 0; kv < hkv; ++kv) {
      std::vector<Unit> u;
      for (int64_t r = 0; r < geos[s].Tm; ++r)
        for (int32_t j = 0; j < grp; ++j)
          u.push_back({(int32_t)s, kv * grp + j, (int32_t)r, geos[s].last_tile(r) + 1});
      for (auto& x : u) total += x.cost;
      if (!u.empty()) groups.push_back(std::move(u));
    }
  }
  const int64_t half_share = std::max<int64_t>(1, total / (2 * kNumXcd));
  for (auto& u : groups) {
    std::stable_sort(u.begin(), u.end(), [](const Unit& a, const Unit& b) { return a.cost > b.cost; });
    int64_t c = 0;
    for (auto& x : u) c += x.cost;
    const int64_t k = std::max<int64_t>(1, std::min<int64_t>((int64_t)u.size(), (c + half_share - 1) / half_share));
    std::vector<std::vector<Unit>> p(k);
    for (size_t i = 0; i < u.size(); ++i) p[i % k].push_back(u[i]);
    for (auto& x : p) parts.push_back(std::move(x));
  }
  std::vector<int64_t> part_cost(parts.size());
  for (size_t i = 0; i < parts.size(); ++i)
    for (auto& x : parts[i]) part_cost[i] += x.cost;
  std::vector<size_t> idx(parts.size());
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](size_t a, size_t b) { return part_cost[a] > part_cost[b]; });
  std::vector<std::vector<Unit>> die(kNumXcd);
  std::vector<int64_t> load(kNumXcd, 0);
  for (size_t i : idx) {
    const int d = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    load[d] += part_cost[i];
    die[d].insert(die[d].end(), parts[i].begin(), parts[i].end());
  }
  // Each die's queue keeps its parts contiguous (largest part first; a part's
  // units longest first): the units in flight on a die then share one or two
  // (sequence, KV head) K/V streams, which stay in that die's L2, and the
  // short units at the end of each part fill the die while the next part's
  // long ones start.
  size_t longest = 0;
  for (auto& q : die) longest = std::max(longest, q.size());
  std::vector<Unit> out;
  out.reserve(longest * kNumXcd);
  for (size_t i = 0; i < longest; ++i)
    for (int d = 0; d < kNumXcd; ++d)
      out.push_back(i < die[d].size() ? die[d][i] : Unit{-1, 0, 0, 0});
  // drop trailing padding
  while (!out.empty() && out.back().seq < 0) out.pop_back();
  return out;
}

int check_plan_args(const int32_t* cu, int32_t batch, int32_t hq, int32_t hkv, int32_t head_dim) {
  int rc = check_cu_seqlens(cu, batch);
  if (rc) return rc;
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0)
    return fail(TILEMIX_EINVAL, "need Hq > 0, Hkv > 0 and Hq %% Hkv == 0 (Hq=%d, Hkv=%d)", hq, hkv);
  if (hq > 32767) return fail(TILEMIX_EINVAL, "Hq=%d exceeds 32767", hq);
  if (head_dim != 64 && head_dim != 128)
    return fail(TILEMIX_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  for (int32_t s = 0; s < batch; ++s)
    if (geometry(cu[s + 1] - cu[s]).Tm > 65535)
      return fail(TILEMIX_EINVAL, "sequence %d is too long (more than 65535 query tiles)", s);
  return TILEMIX_OK;
}

}  // namespace

}  // namespace tilemix

using namespace tilemix;

extern "C" {

const char* tilemix_last_error(void) { return last_error(); }

int tilemix_query_sizes(const int32_t* cu_seqlens_h, int32_t batch, int64_t* total_tokens,
                        int64_t* total_q_tiles, int64_t* total_k_tiles) {
  clear_error();
  int rc = check_cu_seqlens(cu_seqlens_h, batch);
  if (rc) return rc;
  int64_t tm = 0, tn = 0;
  for (int32_t s = 0; s < batch; ++s) {
    const SeqGeo g = geometry(cu_seqlens_h[s + 1] - cu_seqlens_h[s]);
    tm += g.Tm;
    tn += g.Tn;
  }
  if (total_tokens) *total_tokens = cu_seqlens_h[batch];
  if (total_q_tiles) *total_q_tiles = tm;
  if (total_k_tiles) *total_k_tiles = tn;
  return TILEMIX_OK;
}

int tilemix_build_routing(const int32_t* cu_seqlens_h, int32_t batch, int32_t num_kv_heads,
                          int32_t tmpl, int32_t coverage_bp, uint64_t seed, uint64_t* words_h,
                          int32_t* g_h, int64_t* int8_groups_h, int64_t* legal_groups_h) {
  clear_error();
  int rc = check_cu_seqlens(cu_seqlens_h, batch);
  if (rc) return rc;
  if (num_kv_heads <= 0) return fail(TILEMIX_EINVAL, "num_kv_heads must be > 0");
  if (tmpl < TILEMIX_BAND || tmpl > TILEMIX_SPTRANS)
    return fail(TILEMIX_EINVAL, "unknown template id %d", tmpl);
  if (coverage_bp < 0 || coverage_bp > 10000)
    return fail(TILEMIX_EINVAL, "coverage_bp must be in [0, 10000] (got %d)", coverage_bp);
  int64_t total_tm = 0;
  for (int32_t s = 0; s < batch; ++s) total_tm += geometry(cu_seqlens_h[s + 1] - cu_seqlens_h[s]).Tm;
  if (total_tm > 0 && words_h == nullptr) return fail(TILEMIX_EINVAL, "words_h is NULL");
  try {
    int64_t off = 0;
    for (int32_t s = 0; s < batch; ++s) {
      const SeqGeo geo = geometry(cu_seqlens_h[s + 1] - cu_seqlens_h[s]);
      const std::vector<Group> order = template_order(geo, tmpl, seed);
      const int64_t n_legal = (int64_t)order.size();
      const int64_t n8 = (coverage_bp * n_legal + 5000) / 10000;
      std::vector<uint64_t> w(geo.Tm, 0);
      for (int64_t i = n_legal - n8; i < n_legal; ++i) w[order[i].r] |= 1ull << order[i].G;
      if (geo.Tm > 0)  // an empty sequence owns no words (and w.data() may be NULL)
        for (int32_t h = 0; h < num_kv_heads; ++h)
          std::memcpy(words_h + h * total_tm + off, w.data(), geo.Tm * sizeof(uint64_t));
      off += geo.Tm;
      if (g_h) g_h[s] = (int32_t)geo.g;
      if (int8_groups_h) int8_groups_h[s] = n8;
      if (legal_groups_h) legal_groups_h[s] = n_legal;
    }
  } catch (const std::exception& e) {
    return fail(TILEMIX_EINVAL, "routing build failed: %s", e.what());
  }
  return TILEMIX_OK;
}

int tilemix_build_routing3(const int32_t* cu_seqlens_h, int32_t batch, int32_t num_kv_heads, int32_t tmpl,
                           int32_t int8_bp, int32_t fp8_bp, uint64_t seed, uint64_t* words_i8_h,
                           uint64_t* words_f8_h, int32_t* g_h, int64_t* int8_groups_h, int64_t* fp8_groups_h,
                           int64_t* legal_groups_h) {
  clear_error();
  int rc = check_cu_seqlens(cu_seqlens_h, batch);
  if (rc) return rc;
  if (num_kv_heads <= 0) return fail(TILEMIX_EINVAL, "num_kv_heads must be > 0");
  if (tmpl < TILEMIX_BAND || tmpl > TILEMIX_SPTRANS)
    return fail(TILEMIX_EINVAL, "unknown template id %d", tmpl);
  if (int8_bp < 0 || fp8_bp < 0 || int8_bp + fp8_bp > 10000)
    return fail(TILEMIX_EINVAL, "coverages must be >= 0 with int8_bp + fp8_bp <= 10000 (got %d, %d)", int8_bp,
                fp8_bp);
  int64_t total_tm = 0;
  for (int32_t s = 0; s < batch; ++s) total_tm += geometry(cu_seqlens_h[s + 1] - cu_seqlens_h[s]).Tm;
  if (total_tm > 0 && (words_i8_h == nullptr || words_f8_h == nullptr))
    return fail(TILEMIX_EINVAL, "words_i8_h and words_f8_h must not be NULL");
  try {
    int64_t off = 0;
    for (int32_t s = 0; s < batch; ++s) {
      const SeqGeo geo = geometry(cu_seqlens_h[s + 1] - cu_seqlens_h[s]);
      const std::vector<Group> order = template_order(geo, tmpl, seed);
      const int64_t n = (int64_t)order.size();
      const int64_t n8 = (int8_bp * n + 5000) / 10000;
      const int64_t nboth = ((int64_t)(int8_bp + fp8_bp) * n + 5000) / 10000;
      std::vector<uint64_t> w8(geo.Tm, 0), wf(geo.Tm, 0);
      for (int64_t i = n - n8; i < n; ++i) w8[order[i].r] |= 1ull << order[i].G;
      for (int64_t i = n - nboth; i < n - n8; ++i) wf[order[i].r] |= 1ull << order[i].G;
      for (int32_t h = 0; h < num_kv_heads && geo.Tm > 0; ++h) {
        std::memcpy(words_i8_h + h * total_tm + off, w8.data(), geo.Tm * sizeof(uint64_t));
        std::memcpy(words_f8_h + h * total_tm + off, wf.data(), geo.Tm * sizeof(uint64_t));
      }
      off += geo.Tm;
      if (g_h) g_h[s] = (int32_t)geo.g;
      if (int8_groups_h) int8_groups_h[s] = n8;
      if (fp8_groups_h) fp8_groups_h[s] = nboth - n8;
      if (legal_groups_h) legal_groups_h[s] = n;
    }
  } catch (const std::exception& e) {
    return fail(TILEMIX_EINVAL, "routing build failed: %s", e.what());
  }
  return TILEMIX_OK;
}

int tilemix_build_routing_adaptive(const int32_t* cu_seqlens_h, int32_t batch, int32_t num_kv_heads,
                                   const float* importance_h, int32_t coverage_bp, uint64_t* words_h,
                                   int32_t* g_h, int64_t* int8_groups_h, int64_t* legal_groups_h) {
  clear_error();
  int rc = check_cu_seqlens(cu_seqlens_h, batch);
  if (rc) return rc;
  if (num_kv_heads <= 0) return fail(TILEMIX_EINVAL, "num_kv_heads must be > 0");
  if (coverage_bp < 0 || coverage_bp > 10000)
    return fail(TILEMIX_EINVAL, "coverage_bp must be in [0, 10000] (got %d)", coverage_bp);
  int64_t total_tm = 0;
  for (int32_t s = 0; s < batch; ++s) total_tm += geometry(cu_seqlens_h[s + 1] - cu_seqlens_h[s]).Tm;
  if (total_tm > 0 && (words_h == nullptr || importance_h == nullptr))
    return fail(TILEMIX_EINVAL, "words_h and importance_h must not be NULL");
  try {
    int64_t off = 0;
    std::vector<Group> groups;
    for (int32_t s = 0; s < batch; ++s) {
      const SeqGeo geo = geometry(cu_seqlens_h[s + 1] - cu_seqlens_h[s]);
      groups.clear();
      for (int64_t r = 0; r < geo.Tm; ++r)
        for (int64_t G = 0; G <= geo.last_group(r); ++G) groups.push_back({(int32_t)r, (int32_t)G});
      const int64_t n_legal = (int64_t)groups.size();
      const int64_t n8 = (coverage_bp * n_legal + 5000) / 10000;
      for (int32_t h = 0; h < num_kv_heads; ++h) {
        const float* imp = importance_h + ((int64_t)h * total_tm + off) * TILEMIX_WORD_BITS;
        auto key = [&](const Group& x) { return imp[(int64_t)x.r * TILEMIX_WORD_BITS + x.G]; };
        for (const Group& x : groups)
          if (key(x) != key(x)) return fail(TILEMIX_EINVAL, "importance of sequence %d is NaN", s);
        // least important first; ties by (r, G)
        std::vector<Group> order = groups;
        std::stable_sort(order.begin(), order.end(), [&](const Group& a, const Group& b) {
          const float ka = key(a), kb = key(b);
          if (ka != kb) return ka < kb;
          return a.r != b.r ? a.r < b.r : a.G < b.G;
        });
        uint64_t* w = words_h + (int64_t)h * total_tm + off;
        if (geo.Tm > 0) std::memset(w, 0, geo.Tm * sizeof(uint64_t));
        for (int64_t i = 0; i < n8; ++i) w[order[i].r] |= 1ull << order[i].G;
      }
      off += geo.Tm;
      if (g_h) g_h[s] = (int32_t)geo.g;
      if (int8_groups_h) int8_groups_h[s] = n8;
      if (legal_groups_h) legal_groups_h[s] = n_legal;
    }
  } catch (const std::exception& e) {
    return fail(TILEMIX_EINVAL, "adaptive routing build failed: %s", e.what());
  }
  return TILEMIX_OK;
}

int tilemix_plan_size(const int32_t* cu_seqlens_h, int32_t batch, int32_t hq, int32_t hkv,
                      int32_t head_dim, int64_t* plan_len) {
  clear_error();
  int rc = check_plan_args(cu_seqlens_h, batch, hq, hkv, head_dim);
  if (rc) return rc;
  if (plan_len == nullptr) return fail(TILEMIX_EINVAL, "plan_len is NULL");
  std::vector<SeqGeo> geos;
  for (int32_t s = 0; s < batch; ++s) geos.push_back(geometry(cu_seqlens_h[s + 1] - cu_seqlens_h[s]));
  const auto units = schedule(geos, hq, hkv);
  *plan_len = kHeaderLen + (int64_t)batch * kSeqStride + (int64_t)units.size() * kItemStride;
  return TILEMIX_OK;
}

int tilemix_build_plan(const int32_t* cu_seqlens_h, int32_t batch, int32_t hq, int32_t hkv,
                       int32_t head_dim, int32_t* plan_h, int64_t plan_len) {
  clear_error();
  int rc = check_plan_args(cu_seqlens_h, batch, hq, hkv, head_dim);
  if (rc) return rc;
  if (plan_h == nullptr) return fail(TILEMIX_EINVAL, "plan_h is NULL");
  try {
    std::vector<SeqGeo> geos;
    for (int32_t s = 0; s < batch; ++s) geos.push_back(geometry(cu_seqlens_h[s + 1] - cu_seqlens_h[s]));
    const auto units = schedule(geos, hq, hkv);
    const int64_t need = kHeaderLen + (int64_t)batch * kSeqStride + (int64_t)units.size() * kItemStride;
    if (plan_len < need)
      return fail(TILEMIX_EINVAL, "plan buffer holds %lld int32, needs %lld", (long long)plan_len,
                  (long long)need);
    std::memset(plan_h, 0, need * sizeof(int32_t));
    int64_t tm = 0, tn = 0, max_tm = 0;
    int32_t* seq = plan_h + kHeaderLen;
    for (int32_t s = 0; s < batch; ++s) {
      int32_t* rec = seq + s * kSeqStride;
      rec[kSeqStart] = cu_seqlens_h[s];
      rec[kSeqLen] = (int32_t)geos[s].L;
      rec[kSeqQtOff] = (int32_t)tm;
      rec[kSeqKtOff] = (int32_t)tn;
      rec[kSeqG] = (int32_t)geos[s].g;
      rec[kSeqTm] = (int32_t)geos[s].Tm;
      rec[kSeqTn] = (int32_t)geos[s].Tn;
      tm += geos[s].Tm;
      tn += geos[s].Tn;
      max_tm = std::max(max_tm, geos[s].Tm);
    }
    int32_t* items = seq + (int64_t)batch * kSeqStride;
    for (size_t i = 0; i < units.size(); ++i) {
      items[kItemStride * i] = units[i].seq;
      items[kItemStride * i + 1] = (units[i].head << 16) | units[i].row;
    }
    plan_h[kMagic] = kPlanMagic;
    plan_h[kVersion] = kPlanVersion;
    plan_h[kBatch] = batch;
    plan_h[kHq] = hq;
    plan_h[kHkv] = hkv;
    plan_h[kHeadDim] = head_dim;
    plan_h[kTotalTokens] = batch ? cu_seqlens_h[batch] : 0;
    plan_h[kTotalQTiles] = (int32_t)tm;
    plan_h[kTotalKTiles] = (int32_t)tn;
    plan_h[kNumItems] = (int32_t)units.size();
    plan_h[kSeqOff] = kHeaderLen;
    plan_h[kItemOff] = (int32_t)(kHeaderLen + (int64_t)batch * kSeqStride);
    plan_h[kPlanDies] = kNumXcd;
    plan_h[kMaxTm] = (int32_t)max_tm;
    plan_h[kPlanHash] = (int32_t)plan_hash(plan_h);
  } catch (const std::exception& e) {
    return fail(TILEMIX_EINVAL, "plan build failed: %s", e.what());
  }
  return TILEMIX_OK;
}

}  // extern "C"
