// Per-row top-k over the head-reduced scores (k <= 2048).
//
// The selection order is (score descending, key index ascending): the pages ask
// for a deterministic top-k (CANN LightningIndexerV2 guide, "确定性计算") and the
// TileLang guide's golden takes the largest k, sorted. Each key is mapped to a
// unique 64-bit composite
//     c = (ord(score) << 32) | (0xFFFFFFFF - j)
// where ord() maps float order onto unsigned order (-0 folded onto +0), so the
// wanted set is exactly the k largest composites and no tie needs special care.
//
// One workgroup per output row:
//   1. radix select over c, most significant digit first (11/11/10 bits of the
//      score, then of the index part only when scores tie at the threshold):
//      an LDS histogram per digit, a block scan from the top bucket down to find
//      the bucket that holds the k-th largest, stop as soon as that bucket is
//      taken whole;
//   2. compaction of every key with c >= threshold into LDS (exactly k);
//   3. bitonic sort of the winners, descending, and the write-out
//      (indices, float values, -1 / -inf in unused slots).
// Rows that see at most k keys skip step 1-2 and only sort.
#include "li_internal.h"

namespace li {
namespace {

constexpr int kMaxK = 2048;

__device__ inline uint32_t ord_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float from_ord(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

__device__ inline uint64_t composite(float s, int j) {
  return (uint64_t(ord_bits(s)) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(j));
}

// Exclusive prefix sum over the block (thread order), plus the block total.
template <int NTHR>
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
  constexpr int NW = NTHR / 64;
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
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = s_wave[w];
    if (w < wave) before += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

template <int NTHR>
__global__ __launch_bounds__(NTHR) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ unsigned long long sbuf[kMaxK];
  __shared__ uint32_t s_wave[NTHR / 64];
  __shared__ uint32_t s_sel[4];  // bucket, count above it, bucket count, compaction cursor

  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;

  // sequence of this row: the last record with row_base <= r
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.batches[mid].row_base <= r) lo = mid; else hi = mid - 1;
  }
  const BatchRec br = a.batches[lo];
  const int i = (int)(r - br.row_base);
  const int nv = i < br.s_q ? visible_keys(i, br.s_q, br.s_k, a.sparse_mode) : 0;
  const int K = a.k;
  const int m = nv < K ? nv : K;
  const float* src = a.ws + br.ws_off + (int64_t)i * br.ld;
  int32_t* oi = a.out_idx + r * K;
  float* ov = a.out_val ? a.out_val + r * K : nullptr;

  int P = 1;
  while (P < m) P <<= 1;

  if (nv <= K) {
    for (int j = tid; j < P; j += NTHR) sbuf[j] = j < nv ? composite(src[j], j) : 0ull;
  } else {
    // ---- radix select of the K-th largest composite ----
    const int kShift[6] = {53, 42, 32, 21, 10, 0};
    const int kBits[6] = {11, 11, 10, 11, 11, 10};
    uint64_t prefix = 0;
    int fixed = 64;          // bits >= fixed of every candidate equal those of prefix
    uint32_t need = (uint32_t)K;
    for (int p = 0; p < 6; ++p) {
      const int shift = kShift[p];
      const int nb = 1 << kBits[p];
      const uint32_t mask = (uint32_t)nb - 1u;
      for (int b = tid; b < nb; b += NTHR) hist[b] = 0u;
      __syncthreads();
      const uint64_t hi_pref = fixed >= 64 ? 0ull : (prefix >> fixed);
      for (int j = tid; j < nv; j += NTHR) {
        const uint64_t c = composite(src[j], j);
        if (fixed >= 64 || (c >> fixed) == hi_pref)
          atomicAdd(&hist[(uint32_t)(c >> shift) & mask], 1u);
      }
      __syncthreads();
      // buckets in descending order: thread t owns positions [t*bpt, (t+1)*bpt)
      const int bpt = nb / NTHR;
      uint32_t local = 0;
      for (int q = 0; q < bpt; ++q) local += hist[nb - 1 - (tid * bpt + q)];
      uint32_t total;
      const uint32_t before = block_exclusive_scan<NTHR>(local, s_wave, &total);
      if (before < need && need <= before + local) {
        uint32_t cum = before;
        for (int q = 0; q < bpt; ++q) {
          const int bkt = nb - 1 - (tid * bpt + q);
          const uint32_t h = hist[bkt];
          if (cum + h >= need) {
            s_sel[0] = (uint32_t)bkt;
            s_sel[1] = cum;
            s_sel[2] = h;
            break;
          }
          cum += h;
        }
      }
      __syncthreads();
      const uint32_t bkt = s_sel[0];
      need -= s_sel[1];
      const uint32_t cnt = s_sel[2];
      prefix |= uint64_t(bkt) << shift;
      fixed = shift;
      __syncthreads();
      if (cnt == need) break;
    }
    // ---- compaction: exactly K composites are >= prefix ----
    if (tid == 0) s_sel[3] = 0u;
    __syncthreads();
    for (int j = tid; j < nv; j += NTHR) {
      const uint64_t c = composite(src[j], j);
      if (c >= prefix) {
        const uint32_t pos = atomicAdd(&s_sel[3], 1u);
        if (pos < (uint32_t)K) sbuf[pos] = c;
      }
    }
    for (int j = K + tid; j < P; j += NTHR) sbuf[j] = 0ull;
  }
  __syncthreads();

  // ---- bitonic sort, descending ----
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int x = tid; x < (P >> 1); x += NTHR) {
        const int pos = 2 * x - (x & (stride - 1));
        const int oth = pos + stride;
        const bool desc = (pos & size) == 0;
        const unsigned long long u = sbuf[pos], v = sbuf[oth];
        if ((u < v) == desc) {
          sbuf[pos] = v;
          sbuf[oth] = u;
        }
      }
      __syncthreads();
    }
  }

  // ---- write-out ----
  for (int e = tid; e < K; e += NTHR) {
    int32_t idx = -1;
    float val = -__builtin_huge_valf();
    if (e < m) {
      const unsigned long long c = sbuf[e];
      idx = (int32_t)(0xFFFFFFFFu - (uint32_t)c);
      val = from_ord((uint32_t)(c >> 32));
    }
    oi[e] = idx;
    if (ov) ov[e] = val;
  }
}

}  // namespace

hipError_t launch_topk(const li_problem& p, const TopkArgs& a, hipStream_t s) {
  (void)p;
  if (a.num_rows <= 0) return hipSuccess;
  if (a.k < 1 || a.k > kMaxK) return hipErrorInvalidValue;
  hipLaunchKernelGGL((topk_kernel<512>), dim3((unsigned)a.num_rows), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace li
