// Per-row top-k over the head-reduced scores (k <= 8192).
//
// The selection order is (score descending, key index ascending): the pages ask
// for a deterministic top-k (CANN LightningIndexerV2 guide, "确定性计算") and the
// TileLang guide's golden takes the largest k, sorted. Each key maps to a unique
// 64-bit composite
//     c = (ord(score) << 32) | (0xFFFFFFFF - j)
// where ord() maps float order onto unsigned order (-0 folded onto +0), so the
// wanted set is exactly the k largest composites and the wanted order is
// descending composite order. Every composite is > 0.
//
// One workgroup per top-k record: an output row (or, for split rows below, one
// chunk of a row or one row's chunk lists). Records are grouped by the host into size classes
// (up to 8K, 16K, 32K visible keys, longer), each class sorted longest first so
// that short rows fill the tail of its launch; a class runs a kernel whose NT
// threads keep the row in registers (R scores per thread, loaded as float4) or,
// past 32K keys, re-read it from memory on every pass. Block-wide scans and
// min / max go through DPP lane shifts inside each wave.
//
// Fast path (any row whose scores spread over a finite range):
//   1. min / max of the row (block reduction);
//   2. histogram over 4096 buckets linear in the score between min and max
//      (monotone in the score, so bucket order is score order; the buckets follow
//      the data's range, so they stay short);
//   3. a block scan from the top bucket down finds the bucket t holding the k-th
//      largest and turns the counts into each bucket's output offset;
//   4. every key in a bucket >= t is written to its bucket's segment in LDS
//      (a counting sort by bucket);
//   5. each such key's rank inside its segment (a count of larger composites)
//      gives its final sorted position, where it is stored; keys of bucket t
//      ranked past what is still needed are dropped.
// Fallback (zero or non-finite range, or a bucket >= t holding more than
// kSegMax keys, e.g. many equal scores): MSD radix select over the composite
// with 11/11/10-bit digits (score first, index digits only on ties at the
// threshold), compaction of the k winners into LDS and a bitonic sort.
//
// Split rows: where a problem has too few rows to fill the CUs, the host cuts
// each long row into chunks of at most 8192 keys (each longer than k). A first
// pass selects every chunk's top k (sorted, with values) into a candidate list
// in the workspace, the chunks of a row side by side in key order; a second
// pass selects the row's top k over its lists. The k largest composites of a
// row are among its chunks' k largest, and equal scores in the lists stand in
// key order (chunk order, then index order inside a chunk), so selecting on
// list position and mapping the position back to the key gives the same
// result as the whole row.
//
// Routing options of the ops-transformer issue's forward operator: the blocks
// that are always kept (the first init_num and the last local_num of a row) are
// written first, in ascending order, and the selection above runs over the
// blocks between them for the remaining slots (the KEPT kernels). Every stored
// index gets the batch's output_idx_offset.
#include "li_internal.h"

#include <type_traits>

namespace li {
namespace {

constexpr int kMaxKSmall = 2048;      // k of the default kernels (LDS sized for it)
constexpr int kMaxKLarge = 8192;      // k of the large-k kernels
constexpr int kBuckets = 4096;        // fast-path histogram
constexpr int kRadixBins = 2048;      // fallback digit histogram
constexpr int kSegMax = 64;           // longest bucket segment the rank step takes
// Zero composites after the candidates (at most k + kSegMax of them): the rank
// step of a key may read up to
// kSegMax + 1 slots past the end of its segment (they hold smaller composites
// of later segments, or these zeros, and never count).
constexpr int kBufPad = kSegMax + 4;

// -0 -> +0 (IEEE: -0 + +0 = +0; every other value is unchanged).
__device__ inline float canon(float x) { return x + 0.0f; }

__device__ inline uint32_t ord_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t flip = (uint32_t)((int32_t)u >> 31) | 0x80000000u;
  return u ^ flip;
}

__device__ inline float from_ord(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

// Scores enter as read; -0 is folded onto +0 here, the only place where the
// sign of a zero would matter (bucketing maps both zeros alike).
__device__ inline unsigned long long composite(float s, int j) {
  return ((unsigned long long)ord_bits(canon(s)) << 32) |
         (unsigned long long)(0xFFFFFFFFu - (uint32_t)j);
}

__device__ inline int32_t index_of(unsigned long long c) { return (int32_t)(0xFFFFFFFFu - (uint32_t)c); }

// The fast path's composite for rows of at most 2^20 keys also carries the
// key's bucket b in the top 12 bits of its low word: (ord(score), b, 2^20-1-j).
// Inside a bucket segment the order is the plain composite's (b is common);
// a key of a lower bucket has a lower score, so its composite is lower whatever
// its low word holds.
constexpr uint32_t kIdxMask = (1u << 20) - 1;
__device__ inline unsigned long long bucket_composite(float s, int b, int j) {
  return ((unsigned long long)ord_bits(canon(s)) << 32) |
         (unsigned long long)(((uint32_t)b << 20) | (kIdxMask - (uint32_t)j));
}
__device__ inline int bucket_of(unsigned long long c) { return (int)((uint32_t)c >> 20); }
__device__ inline int32_t bucket_index_of(unsigned long long c) {
  return (int32_t)(kIdxMask - ((uint32_t)c & kIdxMask));
}

// Where a record's result goes: output slots idx[d] / val[d] (val may be null).
// A key's stored index is its position in the record's input, mapped through
// gather when the input is a split row's candidate lists, plus off.
struct Out {
  int32_t* idx;
  float* val;
  const int32_t* gather;
  int32_t off;
  __device__ void put(uint32_t d, unsigned long long c) const { put_key(d, index_of(c), c); }
  __device__ void put_key(uint32_t d, int32_t j, unsigned long long c) const {
    idx[d] = (gather ? gather[j] : j) + off;
    if (val) val[d] = from_ord((uint32_t)(c >> 32));
  }
};

// W16: bucket counters are 16-bit halves of 32-bit words (rows of at most 65535
// keys), else whole 32-bit words. The words are contiguous: a bucket's word
// address is then a shift of its index (the hot histogram and counting-sort
// loops spend two VALU operations on it), and the block scan, where each thread
// walks a run of consecutive words, reads and writes them with 16-byte LDS
// accesses. (A pad word after every eight made the scan conflict-free but cost
// three more VALU operations per key and 6% of the top-k time.)
template <bool W16> constexpr int kCounterWords = W16 ? kBuckets / 2 : kBuckets;

template <int NT, bool W16, int KMAX>
struct Smem {
  alignas(16) uint32_t cnt[kCounterWords<W16>];   // histogram, offsets; radix digits
  unsigned long long buf[KMAX + kSegMax + kBufPad];  // composites grouped by bucket
  uint32_t s_wave[NT / 64];
  float s_red[2 * (NT / 64)];
  uint32_t s_sel[4];
};
static_assert(kBuckets / 2 >= kRadixBins, "radix digits reuse the histogram words");

template <bool W16>
struct Counters {
  uint32_t* w;
  __device__ uint32_t& word(int i) const { return w[i]; }
  __device__ uint32_t get(int b) const {
    if constexpr (W16) return (word(b >> 1) >> ((b & 1) << 4)) & 0xFFFFu;
    else return word(b);
  }
  __device__ void add(int b) const {
    if constexpr (W16) atomicAdd(&word(b >> 1), 1u << ((b & 1) << 4));
    else atomicAdd(&word(b), 1u);
  }
  __device__ uint32_t fetch_add(int b) const {
    if constexpr (W16) return (atomicAdd(&word(b >> 1), 1u << ((b & 1) << 4)) >> ((b & 1) << 4)) & 0xFFFFu;
    else return atomicAdd(&word(b), 1u);
  }
};

// Inclusive prefix over the 64 lanes of a wave with DPP: shifts by 1, 2, 4, 8
// inside each 16-lane row, then row 0's / row 2's last lane broadcast into rows
// 1 / 3 and lane 31 into rows 2 and 3. Lanes whose source lies outside the row
// (or whose row is masked off) combine with `id`.
template <int CTRL, int ROWS, typename T, typename Op>
__device__ inline T dpp_step(T x, T id, Op op) {
  const int y = __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, id), __builtin_bit_cast(int, x),
                                            CTRL, ROWS, 0xF, false);
  return op(x, __builtin_bit_cast(T, y));
}

template <typename T, typename Op>
__device__ inline T wave_scan(T x, T id, Op op) {
  x = dpp_step<0x111, 0xF>(x, id, op);   // row_shr:1
  x = dpp_step<0x112, 0xF>(x, id, op);   // row_shr:2
  x = dpp_step<0x114, 0xF>(x, id, op);   // row_shr:4
  x = dpp_step<0x118, 0xF>(x, id, op);   // row_shr:8
  x = dpp_step<0x142, 0xA>(x, id, op);   // row_bcast:15
  x = dpp_step<0x143, 0xC>(x, id, op);   // row_bcast:31
  return x;
}

// Exclusive prefix sum over the block in thread order.
template <int NT>
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t x = wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (w < wave) before += s_wave[w];
  return before + x - v;
}

template <int NT>
__device__ inline void block_minmax(float& lo, float& hi, float* s_red) {
  constexpr int NW = NT / 64;
  lo = wave_scan(lo, __builtin_huge_valf(), [](float a, float b) { return fminf(a, b); });
  hi = wave_scan(hi, -__builtin_huge_valf(), [](float a, float b) { return fmaxf(a, b); });
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 63) {
    s_red[wave] = lo;
    s_red[NW + wave] = hi;
  }
  __syncthreads();
  lo = s_red[0];
  hi = s_red[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    lo = fminf(lo, s_red[w]);
    hi = fmaxf(hi, s_red[NW + w]);
  }
}

// Monotone map of [lo, hi] onto bucket indices 0..kBuckets-1 (one rounding, so
// every pass computes the same bucket for the same score). The clamp covers
// both ends: when |lo| is large against the range, the rounded offset can put
// lo slightly outside [0, kBuckets).
struct Bucketing {
  float scale, off;
  __device__ int operator()(float x) const {
    const int b = (int)fmaf(x, scale, off);
    return min(max(b, 0), kBuckets - 1);
  }
};

// Which keys of a float4 group starting at key j0 take part: e in [beg, end)
// (beg = lo - j0; it matters only when leading keys are left out, KEPT).
template <bool KEPT>
struct GroupRange {
  int beg, end;
  __device__ bool ok(int e) const { return (!KEPT || e >= beg) && e < end; }
};

// The row's scores; keys [lo, n) take part in the selection (lo > 0 only with
// KEPT, when the leading blocks are always kept and so left out). RES: in
// registers, thread t holding the float4 groups t + NT*v (v < R/4), i.e. key
// 4*(t + NT*v) + e in x[4v + e]. Otherwise they are streamed from memory on
// every pass, with the same key-to-thread map.
template <int NT, int R, bool RES, bool KEPT>
struct Row {
  static_assert(R % 4 == 0, "whole float4 groups per thread");
  const float* src;   // 16-byte aligned, readable up to the float4 group holding key n-1
  int n;
  int lo_;
  float x[RES ? R : 4];

  __device__ int lo() const { return KEPT ? lo_ : 0; }
  __device__ int count() const { return n - lo(); }

  __device__ inline float4 group(int v) const {   // float4 group v, clamped in range
    const int last = (n - 1) >> 2;
    return reinterpret_cast<const float4*>(src)[v < last ? v : last];
  }

  __device__ inline void load() {
    if constexpr (RES) {
#pragma unroll
      for (int v = 0; v < R / 4; ++v) {
        if (4 * NT * v >= n) break;   // uniform
        const float4 g = group(threadIdx.x + NT * v);
        x[4 * v] = g.x;
        x[4 * v + 1] = g.y;
        x[4 * v + 2] = g.z;
        x[4 * v + 3] = g.w;
      }
    }
  }

  // f(x[4], first key, GroupRange) for every float4 group that holds keys in
  // [lo, n).
  template <typename F>
  __device__ inline void each4(F&& f) const {
    if constexpr (RES) {
#pragma unroll
      for (int v = 0; v < R / 4; ++v) {
        if (4 * NT * v >= n) break;   // uniform
        const int j0 = 4 * (threadIdx.x + NT * v);
        const float g[4] = {x[4 * v], x[4 * v + 1], x[4 * v + 2], x[4 * v + 3]};
        if (j0 < n && (!KEPT || j0 + 4 > lo_)) f(g, j0, GroupRange<KEPT>{lo() - j0, n - j0});
      }
    } else {
      constexpr int kBatch = 4;   // float4 groups in flight per thread
      for (int v0 = threadIdx.x; 4 * v0 < n; v0 += kBatch * NT) {
        float4 q[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) q[u] = group(v0 + u * NT);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int j0 = 4 * (v0 + u * NT);
          const float g[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
          if (j0 < n && (!KEPT || j0 + 4 > lo_)) f(g, j0, GroupRange<KEPT>{lo() - j0, n - j0});
        }
      }
    }
  }

  // f(score, key) for every key in [lo, n). Groups that lie wholly inside
  // (known for the whole block) skip the per-key bound test.
  template <typename F>
  __device__ inline void each(F&& f) const {
    if constexpr (RES) {
#pragma unroll
      for (int v = 0; v < R / 4; ++v) {
        if (4 * NT * v >= n) break;   // uniform
        const int j0 = 4 * (threadIdx.x + NT * v);
        if ((!KEPT || 4 * NT * v >= lo_) && 4 * NT * (v + 1) <= n) {  // uniform
#pragma unroll
          for (int e = 0; e < 4; ++e) f(x[4 * v + e], j0 + e);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if ((!KEPT || j0 + e >= lo_) && j0 + e < n) f(x[4 * v + e], j0 + e);
        }
      }
    } else {
      constexpr int kBatch = 4;   // float4 groups in flight per thread
      for (int v0 = threadIdx.x; 4 * v0 < n; v0 += kBatch * NT) {
        float4 g[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) g[u] = group(v0 + u * NT);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int j0 = 4 * (v0 + u * NT);
          const float s[4] = {g[u].x, g[u].y, g[u].z, g[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if ((!KEPT || j0 + e >= lo_) && j0 + e < n) f(s[e], j0 + e);
        }
      }
    }
  }
};

// Unused output slots [m, K): index -1, value -inf.
__device__ inline void fill_tail(int m, int K, const Out& out, int nt) {
  for (int e = m + (int)threadIdx.x; e < K; e += nt) {
    out.idx[e] = -1;
    if (out.val) out.val[e] = -__builtin_huge_valf();
  }
}

// Fast path; returns false (before writing any output) if it cannot handle the row.
// The histogram words must be zero on entry.
template <int NT, int R, bool RES, bool KEPT, bool W16, int KMAX>
__device__ bool select_by_buckets(const Row<NT, R, RES, KEPT>& row, float lo, float hi, int K, int m,
                                  const Out& out, Smem<NT, W16, KMAX>& sm) {
  const int tid = threadIdx.x;
  const int n = row.count();
  const float range = hi - lo;
  if (!(hi > lo) || !(range <= 3.0e38f)) return false;
  const float scale = (float)kBuckets / range;
  if (!(scale <= 3.0e38f)) return false;
  const Bucketing bucket{scale, -lo * scale};
  const Counters<W16> cnt{sm.cnt};

  row.each([&](float x, int) { cnt.add(bucket(x)); });
  __syncthreads();

  // Thread t owns the counter words of buckets kBuckets-1 - (t*BPT + q), a
  // descending run of WPT words kept in registers through the scan.
  constexpr int BPT = kBuckets / NT;
  constexpr int BPW = W16 ? 2 : 1;          // buckets per counter word
  constexpr int WPT = BPT / BPW;
  static_assert(BPT % 2 == 0, "whole 16-bit counter pairs per thread");
  // word of the thread's q-th bucket pair (descending): covers buckets
  // kBuckets-1 - (tid*BPT + BPW*q) and, for W16, the one below it
  const int w_top = kCounterWords<W16> - 1 - tid * WPT;
  uint32_t word[WPT];
  uint32_t local = 0;
#pragma unroll
  for (int q = 0; q < WPT; ++q) {
    word[q] = cnt.word(w_top - q);
    local += W16 ? (word[q] >> 16) + (word[q] & 0xFFFFu) : word[q];
  }
  const uint32_t before = block_exclusive_scan<NT>(local, sm.s_wave);
  // Counts in descending bucket order: for W16 the high half (odd bucket) first.
  auto count_at = [&](int q, int h) -> uint32_t {   // h = 0: higher bucket of the word
    if constexpr (W16) return h == 0 ? word[q] >> 16 : word[q] & 0xFFFFu;
    else return word[q];
  };
  if (n <= K) {
    if (tid == 0) {
      sm.s_sel[0] = 0u;           // every bucket is taken whole
      sm.s_sel[1] = 0xFFFFFFFFu;
    }
  } else if (before < (uint32_t)K && (uint32_t)K <= before + local) {
    uint32_t cum = before;
#pragma unroll
    for (int q = 0; q < WPT; ++q)
#pragma unroll
      for (int h = 0; h < BPW; ++h) {
        const uint32_t c = count_at(q, h);
        if (cum < (uint32_t)K && (uint32_t)K <= cum + c) {
          sm.s_sel[0] = (uint32_t)(kBuckets - 1 - (tid * BPT + BPW * q + h));
          sm.s_sel[1] = (uint32_t)K - cum;
        }
        cum += c;
      }
  }
  __syncthreads();
  const int t = (int)sm.s_sel[0];
  const uint32_t need = sm.s_sel[1];
  // Counts become exclusive offsets from the top bucket (16-bit fields are each
  // written on their own, so a field that wraps below t cannot spill into its
  // neighbour; only buckets >= t are used, and their offsets stay below
  // K + kSegMax). Track the largest segment at or above t.
  uint32_t cum = before, big = 0;
#pragma unroll
  for (int q = 0; q < WPT; ++q) {
    const int b_hi = kBuckets - 1 - (tid * BPT + BPW * q);
    if constexpr (W16) {
      const uint32_t c_hi = count_at(q, 0), c_lo = count_at(q, 1);
      cnt.word(w_top - q) = ((cum & 0xFFFFu) << 16) | ((cum + c_hi) & 0xFFFFu);
      cum += c_hi + c_lo;
      if (b_hi >= t && c_hi > big) big = c_hi;
      if (b_hi - 1 >= t && c_lo > big) big = c_lo;
    } else {
      const uint32_t c = count_at(q, 0);
      cnt.word(w_top - q) = cum;
      cum += c;
      if (b_hi >= t && c > big) big = c;
    }
  }
  if (big > (uint32_t)kSegMax) atomicMax(&sm.s_sel[2], big);
  __syncthreads();
  if (sm.s_sel[2] != 0u) return false;

  // Counting sort of the keys of buckets >= t into their bucket segments.
  // Afterwards bucket b's segment is [end(b+1), end(b)) (end(kBuckets) = 0).
  row.each4([&](const float (&x)[4], int j0, auto rng) {
    int b[4];
    uint32_t pos[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {   // all four fetch-adds in flight before any write
      b[e] = bucket(x[e]);
      if (rng.ok(e) && b[e] >= t) pos[e] = cnt.fetch_add(b[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (rng.ok(e) && b[e] >= t) {
        if constexpr (W16) sm.buf[pos[e]] = bucket_composite(x[e], b[e], j0 + e);
        else sm.buf[pos[e]] = composite(x[e], j0 + e);
      }
  });
  __syncthreads();
  const uint32_t ncand = cnt.get(t);
  for (int e = tid; e < kBufPad; e += NT) sm.buf[ncand + e] = 0ull;
  __syncthreads();

  // Rank every grouped key inside its segment and store it at its sorted
  // position. Four candidates per thread are ranked together; each step reads
  // two consecutive slots of each segment. Slots past a segment's end hold
  // smaller composites (later segments, or the zero pad), so they never count
  // and need no mask.
  for (uint32_t p0 = tid; p0 < ncand; p0 += 4 * NT) {
    unsigned long long me[4];
    uint32_t s0[4], s1[4], rank[4];
    int bk[4];
    uint32_t len = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t p = p0 + u * NT;
      me[u] = sm.buf[p < ncand ? p : 0];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (W16) bk[u] = bucket_of(me[u]);
      else bk[u] = bucket(from_ord((uint32_t)(me[u] >> 32)));
      s0[u] = bk[u] == kBuckets - 1 ? 0u : cnt.get(bk[u] + 1);
      s1[u] = p0 + u * NT < ncand ? cnt.get(bk[u]) : s0[u];
      rank[u] = 0;
      len = max(len, s1[u] - s0[u]);
    }
    for (uint32_t i = 0; i < len; i += 2) {
      unsigned long long v[4][2];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 2; ++w) v[u][w] = sm.buf[s0[u] + i + w];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 2; ++w) rank[u] += v[u][w] > me[u] ? 1u : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (s0[u] < s1[u] && !(bk[u] == t && rank[u] >= need)) {
        if constexpr (W16) out.put_key(s0[u] + rank[u], bucket_index_of(me[u]), me[u]);
        else out.put(s0[u] + rank[u], me[u]);
      }
    }
  }
  fill_tail(m, K, out, NT);
  return true;
}

// Fallback: exact radix select over the composite, then bitonic sort.
template <int NT, int R, bool RES, bool KEPT, bool W16, int KMAX>
__device__ void select_by_radix(const Row<NT, R, RES, KEPT>& row, int K, int m, const Out& out,
                                Smem<NT, W16, KMAX>& sm) {
  const int tid = threadIdx.x;
  const int n = row.count();
  uint32_t* cnt = sm.cnt;   // kRadixBins 32-bit counters
  int P = 1;
  while (P < m) P <<= 1;
  if (n <= K) {
    row.each([&](float x, int j) { sm.buf[j - row.lo()] = composite(x, j); });
    for (int j = n + tid; j < P; j += NT) sm.buf[j] = 0ull;
  } else {
    const int kShift[6] = {53, 42, 32, 21, 10, 0};
    const int kBits[6] = {11, 11, 10, 11, 11, 10};
    unsigned long long prefix = 0;
    int fixed = 64;
    uint32_t need = (uint32_t)K;
    for (int p = 0; p < 6; ++p) {
      const int shift = kShift[p];
      const int nb = 1 << kBits[p];
      const uint32_t mask = (uint32_t)nb - 1u;
      for (int b = tid; b < nb; b += NT) cnt[b] = 0u;
      __syncthreads();
      const unsigned long long hp = fixed >= 64 ? 0ull : (prefix >> fixed);
      row.each([&](float x, int j) {
        const unsigned long long cv = composite(x, j);
        if (fixed >= 64 || (cv >> fixed) == hp)
          atomicAdd(&cnt[(uint32_t)(cv >> shift) & mask], 1u);
      });
      __syncthreads();
      // Digit buckets nb-1 .. 0 split into NT runs (nb >= NT: 1024 and 2048 buckets).
      const int bpt = nb / NT;
      uint32_t local = 0;
      for (int q = 0; q < bpt; ++q) local += cnt[nb - 1 - (tid * bpt + q)];
      const uint32_t before = block_exclusive_scan<NT>(local, sm.s_wave);
      if (before < need && need <= before + local) {
        uint32_t cum = before;
        for (int q = 0; q < bpt; ++q) {
          const int bkt = nb - 1 - (tid * bpt + q);
          const uint32_t h = cnt[bkt];
          if (cum + h >= need) {
            sm.s_sel[0] = (uint32_t)bkt;
            sm.s_sel[1] = cum;
            sm.s_sel[2] = h;
            break;
          }
          cum += h;
        }
      }
      __syncthreads();
      const uint32_t bkt = sm.s_sel[0];
      need -= sm.s_sel[1];
      const uint32_t cnt_t = sm.s_sel[2];
      prefix |= (unsigned long long)bkt << shift;
      fixed = shift;
      __syncthreads();
      if (cnt_t == need) break;
    }
    if (tid == 0) sm.s_sel[3] = 0u;
    __syncthreads();
    row.each([&](float x, int j) {
      const unsigned long long cv = composite(x, j);
      if (cv >= prefix) {
        const uint32_t pos = atomicAdd(&sm.s_sel[3], 1u);
        if (pos < (uint32_t)K) sm.buf[pos] = cv;
      }
    });
    for (int j = K + tid; j < P; j += NT) sm.buf[j] = 0ull;
  }
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int x = tid; x < (P >> 1); x += NT) {
        const int pos = 2 * x - (x & (stride - 1));
        const int oth = pos + stride;
        const bool desc = (pos & size) == 0;
        const unsigned long long u = sm.buf[pos], v = sm.buf[oth];
        if ((u < v) == desc) {
          sm.buf[pos] = v;
          sm.buf[oth] = u;
        }
      }
      __syncthreads();
    }
  }
  for (int e = tid; e < m; e += NT) out.put(e, sm.buf[e]);
  fill_tail(m, K, out, NT);
}

// One workgroup per record of one size class: record first + blockIdx.x; the
// record's kind says where its scores come from and where its result goes.
// W16 (16-bit bucket counters) is used only for rows of at most 65535 keys.
// A row's latency is a chain of dependent LDS and memory steps, so throughput
// comes from rows in flight: the 256-thread kernel (every row up to 8K keys, in
// one launch) is held to the register budget of five workgroups per CU.
template <int NT, int R, bool RES, bool KEPT, bool W16, int KMAX>
__global__ __launch_bounds__(NT, (NT == 256 && KMAX == kMaxKSmall) ? 5 : 1)
void topk_kernel(TopkArgs a, int first) {
  __shared__ Smem<NT, W16, KMAX> sm;
  const RowRec rr = a.rows[first + blockIdx.x];
  const int nb = rr.n;
  Out out;
  if (rr.kind == kRowChunk) {
    out = Out{a.cand_idx + rr.out_off, a.cand_val + rr.out_off, nullptr, rr.idx_offset};
  } else {
    out = Out{a.out_idx + rr.out_off, a.out_val ? a.out_val + rr.out_off : nullptr,
              rr.kind == kRowMerge ? a.cand_idx + (rr.ws_off - a.cand_val_off) : nullptr,
              rr.idx_offset};
  }
  const float* src = a.ws + rr.ws_off;
  int K = a.k;
  Row<NT, R, RES, KEPT> row;
  row.src = src;
  row.n = nb;
  row.lo_ = 0;
  if constexpr (KEPT) {
    // Blocks always kept: [0, a1) and [b0, nb). They take the first output
    // slots in ascending order; the selection runs over [a1, b0) for the rest.
    const int a1 = min(a.init_num, nb);
    const int b0 = max(a1, nb - a.local_num);
    const int kept = a1 + (nb - b0);
    for (int e = threadIdx.x; e < kept; e += NT) {
      const int j = e < a1 ? e : b0 + (e - a1);
      out.idx[e] = j + out.off;
      if (out.val) out.val[e] = canon(src[j]);
    }
    out.idx += kept;
    if (out.val) out.val += kept;
    K -= kept;
    row.n = b0;
    row.lo_ = a1;
  }
  const int n = row.count();
  const int m = n < K ? n : K;
  if (m == 0) {
    fill_tail(0, K, out, NT);
    return;
  }
  row.load();
  // Clear the histogram while the row loads.
  for (int w = threadIdx.x; w < (int)(sizeof(sm.cnt) / 4); w += NT) sm.cnt[w] = 0u;
  if (threadIdx.x == 0) sm.s_sel[2] = 0u;
  float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
  row.each([&](float x, int) {
    lo = fminf(lo, x);
    hi = fmaxf(hi, x);
  });
  block_minmax<NT>(lo, hi, sm.s_red);
  const bool fast = (!W16 || n <= 65535) &&
                    select_by_buckets<NT, R, RES, KEPT, W16, KMAX>(row, lo, hi, K, m, out, sm);
  if (!fast) {
    __syncthreads();
    select_by_radix<NT, R, RES, KEPT, W16, KMAX>(row, K, m, out, sm);
  }
}

template <int NT, int R, bool RES, bool W16, int KMAX, bool KEPT>
hipError_t launch_class(const TopkArgs& a, int c, hipStream_t s) {
  const int first = a.row_class[c];
  const int count = a.row_class[c + 1] - first;
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL((topk_kernel<NT, R, RES, KEPT, W16, KMAX>), dim3((unsigned)count), dim3(NT),
                     0, s, a, first);
  return hipGetLastError();
}

// Both passes in order (the second reads the candidate lists the first wrote);
// inside a pass one launch per non-empty class.
template <int KMAX, bool KEPT>
hipError_t launch_all(const TopkArgs& a, hipStream_t s) {
  hipError_t e;
  for (int q = 0; q < 2; ++q) {
    const int c0 = q * kTopkClasses;
    if ((e = launch_class<256, 32, true, true, KMAX, KEPT>(a, c0, s)) != hipSuccess) return e;
    if ((e = launch_class<512, 32, true, true, KMAX, KEPT>(a, c0 + 1, s)) != hipSuccess) return e;
    if ((e = launch_class<1024, 32, true, true, KMAX, KEPT>(a, c0 + 2, s)) != hipSuccess) return e;
    if ((e = launch_class<1024, 4, false, false, KMAX, KEPT>(a, c0 + 3, s)) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <bool KEPT>
hipError_t launch_k(const TopkArgs& a, hipStream_t s) {
  return a.k <= kMaxKSmall ? launch_all<kMaxKSmall, KEPT>(a, s) : launch_all<kMaxKLarge, KEPT>(a, s);
}

}  // namespace

hipError_t launch_topk(const li_problem& p, const TopkArgs& a, hipStream_t s) {
  (void)p;
  if (a.k < 1 || a.k > kMaxKLarge) return hipErrorInvalidValue;
  // Resident capacities NT*R must equal the class limits kTopkClassKeys.
  static_assert(256 * 32 == kTopkClassKeys[0] && 512 * 32 == kTopkClassKeys[1] &&
                    1024 * 32 == kTopkClassKeys[2],
                "class capacities");
  static_assert(kTopkClassThreads[0] == 256 && kTopkClassThreads[1] == 512 &&
                    kTopkClassThreads[2] == 1024 && kTopkClassThreads[3] == 1024,
                "class thread counts");
  return (a.init_num > 0 || a.local_num > 0) ? launch_k<true>(a, s) : launch_k<false>(a, s);
}

}  // namespace li
