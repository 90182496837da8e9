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
// One 256-thread workgroup per output row. Rows of up to R*256 keys stay in
// registers for every pass ("resident"); longer rows are re-read from memory.
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
//      segments are short) gives its final sorted position; keys of bucket t
//      ranked past what is still needed are dropped; the sorted winners are
//      permuted in LDS and written out with coalesced stores.
// Fallback (zero or non-finite range, or a bucket >= t holding more than
// kSegMax keys, e.g. many equal scores): MSD radix select over the composite
// with 11/11/10-bit digits (score first, index digits only on ties at the
// threshold), compaction of the k winners into LDS and a bitonic sort.
#include "li_internal.h"

namespace li {
namespace {

constexpr int kMaxK = 2048;
constexpr int kThreads = 256;
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

// Exclusive prefix sum over the block in thread order.
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave) {
  constexpr int NW = kThreads / 64;
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
  __syncthreads();
  return before + x - v;
}

__device__ inline void block_minmax(float& lo, float& hi, float* s_red) {
  constexpr int NW = kThreads / 64;
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
  __syncthreads();
}

struct Smem {
  uint32_t cnt[kBuckets + 64];           // bucket counts / offsets (+ one dummy per lane)
  unsigned long long buf[kBufCap + 64];  // composites by bucket (+ one sink per lane)
  uint32_t s_wave[kThreads / 64];
  float s_red[2 * (kThreads / 64)];
  uint32_t s_sel[8];
};

// Monotone map of [lo, hi] onto bucket indices 0..kBuckets-1 (one rounding, so
// every pass computes the same bucket for the same score).
struct Bucketing {
  float scale, off;
  __device__ int operator()(float x) const {
    const int b = (int)fmaf(x, scale, off);
    return b < kBuckets - 1 ? b : kBuckets - 1;
  }
};

// The row's scores: in registers (R per thread, element j = tid + r*kThreads)
// when RES, else streamed from memory on every pass.
template <int R, bool RES>
struct Row {
  const float* src;
  int n;
  float x[RES ? R : 1];

  // f(x, j, slot) for every element j < n (slot is the register slot if RES).
  template <typename F>
  __device__ inline void each(F&& f) const {
    if constexpr (RES) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (r * kThreads >= n) break;                 // uniform: no element left
        const int j = threadIdx.x + r * kThreads;
        if (j < n) f(x[r], j, r);
      }
    } else {
      // Streamed: batches of kBatch independent loads keep many requests in flight.
      constexpr int kBatch = 8;
      for (int j0 = threadIdx.x; j0 < n; j0 += kBatch * kThreads) {
        float v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int j = j0 + u * kThreads;
          v[u] = j < n ? src[j] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int j = j0 + u * kThreads;
          if (j < n) f(canon(v[u]), j, 0);
        }
      }
    }
  }
};

// Fast path; returns false (before writing any output) if it cannot handle the row.
template <int R, bool RES>
__device__ bool select_by_buckets(const Row<R, RES>& row, float lo, float hi, int K, int m,
                                  int32_t* oi, float* ov, Smem& sm) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int n = row.n;
  const float range = hi - lo;
  if (!(hi > lo) || !(range <= 3.0e38f)) return false;
  const float scale = (float)kBuckets / range;
  if (!(scale <= 3.0e38f)) return false;
  const Bucketing bucket{scale, -lo * scale};

  for (int b = tid; b < kBuckets + 64; b += kThreads) sm.cnt[b] = 0u;
  if (tid == 0) sm.s_sel[2] = 0u;
  __syncthreads();

  // Histogram. Resident rows keep each slot's bucket for the scatter pass.
  int bk[RES ? R : 1];
  if constexpr (RES) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r * kThreads >= n) break;
      const int j = tid + r * kThreads;
      bk[r] = j < n ? bucket(row.x[r]) : kBuckets + lane;
      atomicAdd(&sm.cnt[bk[r]], 1u);
    }
  } else {
    row.each([&](float x, int, int) { atomicAdd(&sm.cnt[bucket(x)], 1u); });
  }
  __syncthreads();

  // Thread t owns buckets kBuckets-1 - (t*BPT + q), i.e. a descending run.
  constexpr int BPT = kBuckets / kThreads;
  uint32_t c[BPT];
  uint32_t local = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    c[q] = sm.cnt[kBuckets - 1 - (tid * BPT + q)];
    local += c[q];
  }
  const uint32_t before = block_exclusive_scan(local, sm.s_wave);
  if (n <= K) {
    if (tid == 0) {
      sm.s_sel[0] = 0u;           // every bucket is taken whole
      sm.s_sel[1] = 0xFFFFFFFFu;
    }
  } else {
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
  // Counts become exclusive offsets (from the top bucket); largest segment >= t.
  uint32_t cum = before, big = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    const int b = kBuckets - 1 - (tid * BPT + q);
    sm.cnt[b] = cum;
    cum += c[q];
    if (b >= t && c[q] > big) big = c[q];
  }
  if (big > 0) atomicMax(&sm.s_sel[2], big);
  __syncthreads();
  if (sm.s_sel[2] > (uint32_t)kSegMax) return false;

  // Counting sort of the keys of buckets >= t into their bucket segments.
  // Keys that do not take part hit a per-lane dummy counter and sink slot, so
  // the resident loop has no per-slot branch. Afterwards bucket b's segment is
  // [cnt[b+1], cnt[b]) (cnt[kBuckets] taken as 0).
  if constexpr (RES) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r * kThreads >= n) break;
      const int j = tid + r * kThreads;
      const bool take = bk[r] >= t && bk[r] < kBuckets;
      const uint32_t pos = atomicAdd(&sm.cnt[take ? bk[r] : kBuckets + lane], 1u);
      sm.buf[take ? pos : (uint32_t)(kBufCap + lane)] = composite(row.x[r], j);
    }
  } else {
    row.each([&](float x, int j, int) {
      const int b = bucket(x);
      if (b >= t) sm.buf[atomicAdd(&sm.cnt[b], 1u)] = composite(x, j);
    });
  }
  __syncthreads();

  // Rank each grouped key inside its segment: its sorted position is the
  // segment start plus the number of larger composites in the segment.
  const uint32_t ncand = sm.cnt[t];
  constexpr int PER = (kBufCap + kThreads - 1) / kThreads;
  unsigned long long keyv[PER];
  int dest[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const uint32_t p = tid + q * kThreads;
    dest[q] = -1;
    keyv[q] = 0ull;
    if (p < ncand) {
      const unsigned long long me = sm.buf[p];
      const int b = bucket(from_ord((uint32_t)(me >> 32)));
      const uint32_t s0 = b == kBuckets - 1 ? 0u : sm.cnt[b + 1];
      const uint32_t s1 = sm.cnt[b];
      uint32_t rank = 0;
      for (uint32_t u = s0; u < s1; u += 4) {
        const unsigned long long v0 = sm.buf[u];
        const unsigned long long v1 = u + 1 < s1 ? sm.buf[u + 1] : 0ull;
        const unsigned long long v2 = u + 2 < s1 ? sm.buf[u + 2] : 0ull;
        const unsigned long long v3 = u + 3 < s1 ? sm.buf[u + 3] : 0ull;
        rank += (v0 > me) + (v1 > me) + (v2 > me) + (v3 > me);
      }
      if (!(b == t && rank >= need)) dest[q] = (int)(s0 + rank);
      keyv[q] = me;
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < PER; ++q)
    if (dest[q] >= 0) sm.buf[dest[q]] = keyv[q];
  __syncthreads();
  for (int e = tid; e < K; e += kThreads) {
    int32_t idx = -1;
    float val = -__builtin_huge_valf();
    if (e < m) {
      const unsigned long long cv = sm.buf[e];
      idx = (int32_t)(0xFFFFFFFFu - (uint32_t)cv);
      val = from_ord((uint32_t)(cv >> 32));
    }
    oi[e] = idx;
    if (ov) ov[e] = val;
  }
  return true;
}

// Fallback: exact radix select over the composite, then bitonic sort.
template <int R, bool RES>
__device__ void select_by_radix(const Row<R, RES>& row, int K, int m, int32_t* oi, float* ov,
                                Smem& sm) {
  const int tid = threadIdx.x;
  const int n = row.n;
  int P = 1;
  while (P < m) P <<= 1;
  if (n <= K) {
    row.each([&](float x, int j, int) { sm.buf[j] = composite(x, j); });
    for (int j = n + tid; j < P; j += kThreads) sm.buf[j] = 0ull;
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
      for (int b = tid; b < nb; b += kThreads) sm.cnt[b] = 0u;
      __syncthreads();
      const unsigned long long hp = fixed >= 64 ? 0ull : (prefix >> fixed);
      row.each([&](float x, int j, int) {
        const unsigned long long cv = composite(x, j);
        if (fixed >= 64 || (cv >> fixed) == hp)
          atomicAdd(&sm.cnt[(uint32_t)(cv >> shift) & mask], 1u);
      });
      __syncthreads();
      const int bpt = nb / kThreads;
      uint32_t local = 0;
      for (int q = 0; q < bpt; ++q) local += sm.cnt[nb - 1 - (tid * bpt + q)];
      const uint32_t before = block_exclusive_scan(local, sm.s_wave);
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
    row.each([&](float x, int j, int) {
      const unsigned long long cv = composite(x, j);
      if (cv >= prefix) {
        const uint32_t pos = atomicAdd(&sm.s_sel[3], 1u);
        if (pos < (uint32_t)K) sm.buf[pos] = cv;
      }
    });
    for (int j = K + tid; j < P; j += kThreads) sm.buf[j] = 0ull;
  }
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int x = tid; x < (P >> 1); x += kThreads) {
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
  for (int e = tid; e < K; e += kThreads) {
    int32_t idx = -1;
    float val = -__builtin_huge_valf();
    if (e < m) {
      const unsigned long long cv = sm.buf[e];
      idx = (int32_t)(0xFFFFFFFFu - (uint32_t)cv);
      val = from_ord((uint32_t)(cv >> 32));
    }
    oi[e] = idx;
    if (ov) ov[e] = val;
  }
}

template <int R, bool RES>
__device__ void select_row(const float* src, int n, int K, int m, int32_t* oi, float* ov,
                           Smem& sm) {
  Row<R, RES> row;
  row.src = src;
  row.n = n;
  float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
  if constexpr (RES) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r * kThreads >= n) break;
      const int j = threadIdx.x + r * kThreads;
      row.x[r] = j < n ? canon(src[j]) : 0.f;
    }
  }
  row.each([&](float x, int, int) {
    lo = fminf(lo, x);
    hi = fmaxf(hi, x);
  });
  block_minmax(lo, hi, sm.s_red);
  if (!select_by_buckets<R, RES>(row, lo, hi, K, m, oi, ov, sm)) {
    __syncthreads();
    select_by_radix<R, RES>(row, K, m, oi, ov, sm);
  }
}

// One workgroup per row. RES: this launch handles the rows of at most R*256
// visible keys (kept in registers); otherwise it handles the longer rows
// (streamed). Rows of the other kind return at once, so two launches cover
// every row with each kernel compiled for its own register budget.
template <int R, bool RES>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;

  // sequence of this row: the last record with row_base <= r
  int lo_b = 0, hi_b = a.batch - 1;
  while (lo_b < hi_b) {
    const int mid = (lo_b + hi_b + 1) >> 1;
    if (a.batches[mid].row_base <= r) lo_b = mid; else hi_b = mid - 1;
  }
  const BatchRec br = a.batches[lo_b];
  const int i = (int)(r - br.row_base);
  const int n = i < br.s_q ? visible_keys(i, br.s_q, br.s_k, a.sparse_mode) : 0;
  if ((n <= R * kThreads) != RES) return;
  const int K = a.k;
  const int m = n < K ? n : K;
  int32_t* oi = a.out_idx + r * K;
  float* ov = a.out_val ? a.out_val + r * K : nullptr;
  if (n == 0) {
    for (int e = tid; e < K; e += kThreads) {
      oi[e] = -1;
      if (ov) ov[e] = -__builtin_huge_valf();
    }
    return;
  }
  const float* src = a.ws + br.ws_off + (int64_t)i * br.ld;
  select_row<R, RES>(src, n, K, m, oi, ov, sm);
}

}  // namespace

hipError_t launch_topk(const li_problem& p, const TopkArgs& a, hipStream_t s) {
  (void)p;
  if (a.num_rows <= 0) return hipSuccess;
  if (a.k < 1 || a.k > kMaxK) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.num_rows), block(kThreads);
  if (a.max_keys <= 8 * kThreads) {
    hipLaunchKernelGGL((topk_kernel<8, true>), grid, block, 0, s, a);
  } else if (a.max_keys <= 16 * kThreads) {
    hipLaunchKernelGGL((topk_kernel<16, true>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((topk_kernel<32, true>), grid, block, 0, s, a);
    if (a.max_keys > 32 * kThreads) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((topk_kernel<32, false>), grid, block, 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace li
