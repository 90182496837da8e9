// Per-row top-k over the head-reduced scores (k <= 2048).
//
// The selection order is (score descending, key index ascending): the pages ask
// for a deterministic top-k (CANN LightningIndexerV2 guide, "确定性计算") and the
// TileLang guide's golden takes the largest k, sorted. Each key maps to a unique
// 64-bit composite
//     c = (ord(score) << 32) | (0xFFFFFFFF - j)
// where ord() maps float order onto unsigned order (-0 folded onto +0), so the
// wanted set is exactly the k largest composites and the wanted order is
// descending composite order.
//
// One workgroup per output row. Rows are grouped by the host into size classes
// (visible keys); each class runs a kernel whose NT threads keep the row in
// registers (R scores per thread, loaded as float4) or, past 32K keys, re-read
// it from memory on every pass.
//
// Fast path (any row whose scores spread over a finite range):
//   1. min / max of the row (block reduction);
//   2. histogram over 2048 buckets linear in the score between min and max
//      (monotone in the score, so bucket order is score order, and contention on
//      the LDS counters stays low because the buckets follow the data's range);
//   3. a block scan from the top bucket down finds the bucket t holding the k-th
//      largest and turns the counts into each bucket's output offset;
//   4. every key in a bucket >= t is written to its bucket's segment in LDS
//      (a counting sort by bucket);
//   5. each such key's rank inside its segment (a count of larger composites;
//      segments are short) gives its final sorted position, where it is stored;
//      keys of bucket t ranked past what is still needed are dropped.
// Fallback (zero or non-finite range, or a bucket >= t holding more than
// kSegMax keys, e.g. many equal scores): MSD radix select over the composite
// with 11/11/10-bit digits (score first, index digits only on ties at the
// threshold), compaction of the k winners into LDS and a bitonic sort.
#include "li_internal.h"

namespace li {
namespace {

constexpr int kMaxK = 2048;
constexpr int kBuckets = 2048;
constexpr int kSegMax = 64;
constexpr int kBufCap = kMaxK + kSegMax;

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

__device__ inline unsigned long long composite(float s, int j) {
  return ((unsigned long long)ord_bits(s) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)j);
}

__device__ inline int32_t index_of(unsigned long long c) { return (int32_t)(0xFFFFFFFFu - (uint32_t)c); }

template <int NT>
struct Smem {
  uint32_t cnt[kBuckets];                // bucket counts, then offsets
  unsigned long long buf[kBufCap];       // composites grouped by bucket
  uint32_t s_wave[NT / 64];
  float s_red[2 * (NT / 64)];
  uint32_t s_sel[4];
};

// Exclusive prefix sum over the block in thread order.
template <int NT>
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
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
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o));
    hi = fmaxf(hi, __shfl_xor(hi, o));
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
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
    const float f = fmaf(x, scale, off);
    const int b = f > 0.f ? (int)f : 0;
    return b < kBuckets - 1 ? b : kBuckets - 1;
  }
};

// The row's n scores. RES: in registers, thread t holding the float4 groups
// t + NT*v (v < R/4), i.e. key 4*(t + NT*v) + e in x[4v + e]. Otherwise they
// are streamed from memory on every pass, with the same key-to-thread map.
template <int NT, int R, bool RES>
struct Row {
  static_assert(R % 4 == 0, "whole float4 groups per thread");
  const float* src;   // 16-byte aligned, readable up to the float4 group holding key n-1
  int n;
  float x[RES ? R : 4];

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
        x[4 * v] = canon(g.x);
        x[4 * v + 1] = canon(g.y);
        x[4 * v + 2] = canon(g.z);
        x[4 * v + 3] = canon(g.w);
      }
    }
  }

  // f(score, key) for every key < n.
  template <typename F>
  __device__ inline void each(F&& f) const {
    if constexpr (RES) {
#pragma unroll
      for (int v = 0; v < R / 4; ++v) {
        if (4 * NT * v >= n) break;   // uniform
        const int j0 = 4 * (threadIdx.x + NT * v);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j0 + e < n) f(x[4 * v + e], j0 + e);
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
            if (j0 + e < n) f(canon(s[e]), j0 + e);
        }
      }
    }
  }
};

// Unused output slots [m, K): index -1, value -inf.
__device__ inline void fill_tail(int m, int K, int32_t* oi, float* ov, int nt) {
  for (int e = m + (int)threadIdx.x; e < K; e += nt) {
    oi[e] = -1;
    if (ov) ov[e] = -__builtin_huge_valf();
  }
}

// Fast path; returns false (before writing any output) if it cannot handle the row.
template <int NT, int R, bool RES>
__device__ bool select_by_buckets(const Row<NT, R, RES>& row, float lo, float hi, int K, int m,
                                  int32_t* oi, float* ov, Smem<NT>& sm) {
  const int tid = threadIdx.x;
  const int n = row.n;
  const float range = hi - lo;
  if (!(hi > lo) || !(range <= 3.0e38f)) return false;
  const float scale = (float)kBuckets / range;
  if (!(scale <= 3.0e38f)) return false;
  const Bucketing bucket{scale, -lo * scale};

  for (int b = tid; b < kBuckets; b += NT) sm.cnt[b] = 0u;
  if (tid == 0) sm.s_sel[2] = 0u;
  __syncthreads();
  row.each([&](float x, int) { atomicAdd(&sm.cnt[bucket(x)], 1u); });
  __syncthreads();

  // Thread t owns buckets kBuckets-1 - (t*BPT + q), a descending run.
  constexpr int BPT = kBuckets / NT;
  uint32_t c[BPT];
  uint32_t local = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    c[q] = sm.cnt[kBuckets - 1 - (tid * BPT + q)];
    local += c[q];
  }
  const uint32_t before = block_exclusive_scan<NT>(local, sm.s_wave);
  if (n <= K) {
    if (tid == 0) {
      sm.s_sel[0] = 0u;           // every bucket is taken whole
      sm.s_sel[1] = 0xFFFFFFFFu;
    }
  } else if (before < (uint32_t)K && (uint32_t)K <= before + local) {
    uint32_t cum = before;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      if (cum < (uint32_t)K && (uint32_t)K <= cum + c[q]) {
        sm.s_sel[0] = (uint32_t)(kBuckets - 1 - (tid * BPT + q));
        sm.s_sel[1] = (uint32_t)K - cum;
      }
      cum += c[q];
    }
  }
  __syncthreads();
  const int t = (int)sm.s_sel[0];
  const uint32_t need = sm.s_sel[1];
  // Counts become exclusive offsets from the top bucket; largest segment >= t.
  uint32_t cum = before, big = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    const int b = kBuckets - 1 - (tid * BPT + q);
    sm.cnt[b] = cum;
    cum += c[q];
    if (b >= t && c[q] > big) big = c[q];
  }
  if (big > (uint32_t)kSegMax) atomicMax(&sm.s_sel[2], big);
  __syncthreads();
  if (sm.s_sel[2] != 0u) return false;

  // Counting sort of the keys of buckets >= t into their bucket segments.
  // Afterwards bucket b's segment is [cnt[b+1], cnt[b]) (cnt[kBuckets] = 0).
  row.each([&](float x, int j) {
    const int b = bucket(x);
    if (b >= t) sm.buf[atomicAdd(&sm.cnt[b], 1u)] = composite(x, j);
  });
  __syncthreads();

  // Rank every grouped key inside its segment and store it at its sorted
  // position. Four candidates per thread are ranked together so that their
  // LDS reads overlap.
  const uint32_t ncand = sm.cnt[t];
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
      bk[u] = bucket(from_ord((uint32_t)(me[u] >> 32)));
      s0[u] = bk[u] == kBuckets - 1 ? 0u : sm.cnt[bk[u] + 1];
      s1[u] = p0 + u * NT < ncand ? sm.cnt[bk[u]] : s0[u];
      rank[u] = 0;
      len = max(len, s1[u] - s0[u]);
    }
    // Four segment positions of each of the four candidates per step: sixteen
    // independent LDS reads (addresses clamped into the segment, out-of-range
    // positions masked in the compare).
    for (uint32_t i = 0; i < len; i += 4) {
      unsigned long long v[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t at = s0[u] + i + w;
          v[u][w] = sm.buf[at < s1[u] ? at : s0[u]];
        }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          rank[u] += (s0[u] + i + w < s1[u] && v[u][w] > me[u]) ? 1u : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (s0[u] < s1[u] && !(bk[u] == t && rank[u] >= need)) {
        const uint32_t d = s0[u] + rank[u];
        oi[d] = index_of(me[u]);
        if (ov) ov[d] = from_ord((uint32_t)(me[u] >> 32));
      }
    }
  }
  fill_tail(m, K, oi, ov, NT);
  return true;
}

// Fallback: exact radix select over the composite, then bitonic sort.
template <int NT, int R, bool RES>
__device__ void select_by_radix(const Row<NT, R, RES>& row, int K, int m, int32_t* oi, float* ov,
                                Smem<NT>& sm) {
  const int tid = threadIdx.x;
  const int n = row.n;
  int P = 1;
  while (P < m) P <<= 1;
  if (n <= K) {
    row.each([&](float x, int j) { sm.buf[j] = composite(x, j); });
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
      for (int b = tid; b < nb; b += NT) sm.cnt[b] = 0u;
      __syncthreads();
      const unsigned long long hp = fixed >= 64 ? 0ull : (prefix >> fixed);
      row.each([&](float x, int j) {
        const unsigned long long cv = composite(x, j);
        if (fixed >= 64 || (cv >> fixed) == hp)
          atomicAdd(&sm.cnt[(uint32_t)(cv >> shift) & mask], 1u);
      });
      __syncthreads();
      // Digit buckets nb-1 .. 0 split into NT runs (nb >= NT: 1024 and 2048 buckets).
      const int bpt = nb / NT;
      uint32_t local = 0;
      for (int q = 0; q < bpt; ++q) local += sm.cnt[nb - 1 - (tid * bpt + q)];
      const uint32_t before = block_exclusive_scan<NT>(local, sm.s_wave);
      if (before < need && need <= before + local) {
        uint32_t cum = before;
        for (int q = 0; q < bpt; ++q) {
          const int bkt = nb - 1 - (tid * bpt + q);
          const uint32_t h = sm.cnt[bkt];
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
      const uint32_t cnt = sm.s_sel[2];
      prefix |= (unsigned long long)bkt << shift;
      fixed = shift;
      __syncthreads();
      if (cnt == need) break;
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
  for (int e = tid; e < m; e += NT) {
    const unsigned long long cv = sm.buf[e];
    oi[e] = index_of(cv);
    if (ov) ov[e] = from_ord((uint32_t)(cv >> 32));
  }
  fill_tail(m, K, oi, ov, NT);
}

// One workgroup per row of one size class: row record first + blockIdx.x.
template <int NT, int R, bool RES>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a, int first) {
  __shared__ Smem<NT> sm;
  const RowRec rr = a.rows[first + blockIdx.x];
  const BatchRec br = a.batches[rr.b];
  const int i = rr.row - br.row_base;
  const int n = i < br.s_q ? visible_keys(i, br.s_q, br.s_k, a.sparse_mode) : 0;
  const int K = a.k;
  const int m = n < K ? n : K;
  int32_t* oi = a.out_idx + (int64_t)rr.row * K;
  float* ov = a.out_val ? a.out_val + (int64_t)rr.row * K : nullptr;
  if (n == 0) {
    fill_tail(0, K, oi, ov, NT);
    return;
  }
  Row<NT, R, RES> row;
  row.src = a.ws + br.ws_off + (int64_t)i * br.ld;
  row.n = n;
  row.load();
  float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
  row.each([&](float x, int) {
    lo = fminf(lo, x);
    hi = fmaxf(hi, x);
  });
  block_minmax<NT>(lo, hi, sm.s_red);
  if (!select_by_buckets<NT, R, RES>(row, lo, hi, K, m, oi, ov, sm)) {
    __syncthreads();
    select_by_radix<NT, R, RES>(row, K, m, oi, ov, sm);
  }
}

template <int NT, int R, bool RES>
hipError_t launch_class(const TopkArgs& a, int c, hipStream_t s) {
  const int first = a.row_class[c];
  const int count = a.row_class[c + 1] - first;
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL((topk_kernel<NT, R, RES>), dim3((unsigned)count), dim3(NT), 0, s, a, first);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const li_problem& p, const TopkArgs& a, hipStream_t s) {
  (void)p;
  if (a.k < 1 || a.k > kMaxK) return hipErrorInvalidValue;
  // Resident capacities NT*R must equal the class limits kTopkClassKeys.
  static_assert(256 * 8 == kTopkClassKeys[0] && 256 * 16 == kTopkClassKeys[1] &&
                    256 * 32 == kTopkClassKeys[2] && 512 * 32 == kTopkClassKeys[3] &&
                    1024 * 32 == kTopkClassKeys[4],
                "class capacities");
  static_assert(kTopkClassThreads[0] == 256 && kTopkClassThreads[3] == 512 &&
                    kTopkClassThreads[4] == 1024 && kTopkClassThreads[5] == 1024,
                "class thread counts");
  hipError_t e;
  if ((e = launch_class<256, 8, true>(a, 0, s)) != hipSuccess) return e;
  if ((e = launch_class<256, 16, true>(a, 1, s)) != hipSuccess) return e;
  if ((e = launch_class<256, 32, true>(a, 2, s)) != hipSuccess) return e;
  if ((e = launch_class<512, 32, true>(a, 3, s)) != hipSuccess) return e;
  if ((e = launch_class<1024, 32, true>(a, 4, s)) != hipSuccess) return e;
  return launch_class<1024, 4, false>(a, 5, s);
}

}  // namespace li
