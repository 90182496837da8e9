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
//   2. histogram over nb buckets linear in the score between min and max
//      (monotone in the score, so bucket order is score order; the buckets follow
//      the data's range, so they stay short); nb is the row length rounded up
//      to a power of two, at most 4096;
//   3. a block scan from the top bucket down finds the bucket t holding the k-th
//      largest and turns the counts into each bucket's output offset;
//   4. every key in a bucket >= t is written to its bucket's segment in LDS
//      (a counting sort by bucket);
//   5. each such key's rank inside its segment (a count of larger composites)
//      gives its final sorted position, where it is stored if below k (only
//      keys of bucket t can land at k or past it).
// Scores arrive canonical: the score kernel stores x + 0 (no -0, NaNs quiet),
// so composites need no folding of -0 and min / max no NaN quieting.
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
// step of a key reads its segment two slots at a time up to the longest
// segment among the keys its thread ranks together, i.e. up to kSegMax + 1
// slots past the end of its own segment (they hold smaller composites of later
// segments, or these zeros, and never count).
constexpr int kBufPad = kSegMax + 4;

// -0 -> +0 (IEEE: -0 + +0 = +0; every other value is unchanged).
__device__ inline float canon(float x) { return x + 0.0f; }

// min / max as single instructions. The compiler's fminf / fmaxf first quiet
// signalling NaNs in every operand it cannot prove canonical (one more
// instruction per operand); the scores are canonical already (stored as x + 0).
__device__ inline float min_raw(float a, float b) {
  float r;
  asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ inline float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ inline float min3_raw(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ inline float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

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

// The fast path's composite (rows of at most 65535 keys) also carries the
// key's bucket b in the low 12 bits of its low word, the complemented index in
// the high 16: (ord(score), 65535-j, b). s is canonical (as the score kernel
// stores it); rjs = (65535-j) << 16. Inside a bucket segment the order is the
// plain composite's (b is common); a key of a lower bucket has a lower score,
// so its composite is lower whatever its low word holds.
constexpr uint32_t kIdxMask = 0xFFFFu;
__device__ inline unsigned long long bucket_composite(float s, int b, uint32_t rjs) {
  return ((unsigned long long)ord_bits(s) << 32) | (rjs + (uint32_t)b);
}
// (bits 12-15 are zero, so the low half is the bucket: one SDWA operand)
__device__ inline int bucket_of(unsigned long long c) { return (int)((uint32_t)c & 0xFFFFu); }
__device__ inline int32_t bucket_index_of(unsigned long long c) {
  return (int32_t)(kIdxMask - ((uint32_t)c >> 16));
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
  // Fast-path store from the composite's low word lw (65535-j in its high
  // half) through buffer records of k slots: a slot at or past k is dropped by
  // the hardware, and j + off is one subtraction of lw's high half from a
  // uniform constant (records without gather only).
  __device__ void put_rj(__amdgpu_buffer_rsrc_t ridx, __amdgpu_buffer_rsrc_t rval, uint32_t d,
                         uint32_t lw, unsigned long long c) const {
    int32_t v;
    asm("v_sub_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
        : "=v"(v) : "s"(kIdxMask + (uint32_t)off), "v"(lw));
    const int b = (int)(d * 4u);
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)v, ridx, b, 0, 0);
    if (val) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(from_ord((uint32_t)(c >> 32))), rval, b,
                                                   0, 0);
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
  // histogram, offsets; radix digits. The word past the buckets stays zero: it
  // is the end of the (empty) segment above the top bucket.
  alignas(16) uint32_t cnt[kCounterWords<W16> + 4];
  unsigned long long buf[KMAX + kSegMax + kBufPad];  // composites grouped by bucket
  uint32_t s_wave[NT / 64];
  uint32_t s_red[2 * (NT / 64)];
  uint32_t s_sel[4];
};
static_assert(kBuckets / 2 >= kRadixBins, "radix digits reuse the histogram words");

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// acc + (w >> 16) + (w & 0xFFFF) in one instruction (a u16 dot product).
__device__ inline uint32_t add_halves(uint32_t w, uint32_t acc) {
  const u16x2_t one = {1, 1};
  return __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2_t, w), one, acc, false);
}

template <bool W16>
struct Counters {
  uint32_t* w;
  __device__ uint32_t& word(int i) const { return w[i]; }
  __device__ uint32_t get(int b) const {
    if constexpr (W16) return (word(b >> 1) >> ((b & 1) << 4)) & 0xFFFFu;
    else return word(b);
  }
  // (get(b + 1), get(b)). For 16-bit counters these are the two consecutive
  // halfwords at bytes 2b + 2 and 2b (little-endian halves), read as such.
  __device__ void get_pair(int b, uint32_t& up, uint32_t& at) const {
    if constexpr (W16) {
      const uint16_t* h = reinterpret_cast<const uint16_t*>(w);
      at = h[b];
      up = h[b + 1];
    } else {
      at = word(b);
      up = word(b + 1);
    }
  }
  __device__ void add(int b) const {
    if constexpr (W16) atomicAdd(&word(b >> 1), 1u << ((b & 1) << 4));
    else atomicAdd(&word(b), 1u);
  }
  // fetch_add split in two, so that several atomics can be in flight before the
  // first result is used: the raw old word, then the bucket's old count in it.
  template <uint32_t U = 1>
  __device__ uint32_t fetch_add_raw(int b) const {
    if constexpr (W16) return atomicAdd(&word(b >> 1), U << ((b & 1) << 4));
    else return atomicAdd(&word(b), U);
  }
  __device__ uint32_t field(uint32_t raw, int b) const {
    // the field's offset is (b & 1) * 16: v_bfe_u32 reads only the low five
    // bits of b << 4
    if constexpr (W16) return __builtin_amdgcn_ubfe(raw, (uint32_t)b << 4, 16);
    else return raw;
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

// Exclusive prefix sum over the block in thread order. Waves from nw_act on
// must hold v = 0; they skip their scan.
template <int NT>
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, int nw_act = NT / 64) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t x = 0;
  if (wave < nw_act) x = wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (w < wave) before += s_wave[w];
  return before + x - v;
}

template <int NT>
__device__ inline void block_minmax(float& lo, float& hi, uint32_t* s_red) {
  // On order-preserving bits the two reductions are unsigned maxima (of ~ord(lo)
  // and of ord(hi)) with identity 0, so each DPP step is one fused instruction.
  constexpr int NW = NT / 64;
  const auto umax = [](uint32_t a, uint32_t b) { return max(a, b); };
  uint32_t a = wave_scan(~ord_bits(lo), 0u, umax);
  uint32_t b = wave_scan(ord_bits(hi), 0u, umax);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 63) {
    s_red[wave] = a;
    s_red[NW + wave] = b;
  }
  __syncthreads();
  a = s_red[0];
  b = s_red[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    a = max(a, s_red[w]);
    b = max(b, s_red[NW + w]);
  }
  lo = from_ord(~a);
  hi = from_ord(b);
}

// Monotone map of [lo, hi] onto bucket indices 0..nb-1: floor((x - lo) * scale)
// with scale = (nb - 1/2) / (hi - lo). x - lo rounds to a value in [0, hi - lo]
// (rounding is monotone and exact at 0), and (hi - lo) * scale rounds below nb,
// so no clamp is needed; every pass computes the same bucket for a score.
struct Bucketing {
  float scale, lo;
  __device__ int operator()(float x) const { return (int)((x - lo) * scale); }
};

// Which keys of a float4 group starting at key j0 take part: e in [beg, end)
// (beg = lo - j0; it matters only when leading keys are left out, KEPT).
template <bool KEPT>
struct GroupRange {
  int beg, end;
  bool full;   // uniform: every key of the group takes part
  __device__ bool ok(int e) const { return full || ((!KEPT || e >= beg) && e < end); }
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
        if ((!KEPT || 4 * NT * v >= lo_) && 4 * NT * (v + 1) <= n)   // uniform
          f(g, j0, GroupRange<KEPT>{0, 4, true});
        else if (j0 < n && (!KEPT || j0 + 4 > lo_))
          f(g, j0, GroupRange<KEPT>{lo() - j0, n - j0, false});
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
          if (j0 < n && (!KEPT || j0 + 4 > lo_)) f(g, j0, GroupRange<KEPT>{lo() - j0, n - j0, false});
        }
      }
    }
  }

  // Running min / max over the keys in [lo, n) (NaN scores are skipped).
  __device__ inline void minmax(float& mn, float& mx) const {
    constexpr float kInf = __builtin_huge_valf();
    if constexpr (RES) {
#pragma unroll
      for (int v = 0; v < R / 4; ++v) {
        if (4 * NT * v >= n) break;   // uniform
        const float* g = &x[4 * v];
        if ((!KEPT || 4 * NT * v >= lo_) && 4 * NT * (v + 1) <= n) {  // uniform: all in range
          mn = min3_raw(mn, g[0], g[1]);
          mn = min3_raw(mn, g[2], g[3]);
          mx = max3_raw(mx, g[0], g[1]);
          mx = max3_raw(mx, g[2], g[3]);
        } else {
          const int j0 = 4 * (threadIdx.x + NT * v);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool in = (!KEPT || j0 + e >= lo_) && j0 + e < n;
            mn = min_raw(mn, in ? g[e] : kInf);
            mx = max_raw(mx, in ? g[e] : -kInf);
          }
        }
      }
    } else {
      each([&](float s, int) {
        mn = min_raw(mn, s);
        mx = max_raw(mx, s);
      });
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
  // nb buckets: the row length rounded up to a power of two, between one
  // wave's share and kBuckets. Short rows then scan fewer buckets (only the
  // waves that own buckets take part) while their segments stay short; rows of
  // 2K-4K keys keep kBuckets (halving them there lengthened the segments and
  // cost 7% on such rows).
  constexpr int BPT = kBuckets / NT;        // buckets per active thread
  constexpr int BPW = W16 ? 2 : 1;          // buckets per counter word
  constexpr int WPT = BPT / BPW;
  static_assert(BPT % 2 == 0, "whole 16-bit counter pairs per thread");
  constexpr int NB_MIN = BPT * 64;          // the buckets of one wave
  int nb = NB_MIN;
  while (nb < kBuckets && nb < n) nb <<= 1;   // uniform
  const float scale = ((float)nb - 0.5f) / range;
  if (!(scale <= 3.0e38f)) return false;
  const Bucketing bucket{scale, lo};
  const Counters<W16> cnt{sm.cnt};
  // Offsets count bytes of buf (U = 8) where (K + kSegMax) * 8 fits a 16-bit
  // field; the counting sort and the rank step then address buf without a shift.
  constexpr uint32_t U = (!W16 || KMAX <= 2048) ? 8u : 1u;
  static_assert(!W16 || U == 1 || (KMAX + kSegMax) * 8 < 65536, "16-bit byte offsets");
  auto at = [&](uint32_t off) -> unsigned long long& {
    return *reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(sm.buf) + off * (8 / U));
  };

  row.each([&](float x, int) { cnt.add(bucket(x)); });
  __syncthreads();

  // Active thread t (t * BPT < nb; whole waves) owns buckets nb-1 - (t*BPT + q),
  // a descending run of WPT words kept in registers through the scan.
  const bool act = tid * BPT < nb;              // uniform per wave
  const int nw_act = nb / NB_MIN;
  // word of the thread's q-th bucket pair (descending): covers buckets
  // nb-1 - (tid*BPT + BPW*q) and, for W16, the one below it
  const int w_top = nb / BPW - 1 - tid * WPT;
  uint32_t word[WPT];
  uint32_t local = 0;
#pragma unroll
  for (int q = 0; q < WPT; ++q) word[q] = 0;
  if (act) {
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      word[q] = cnt.word(w_top - q);
      local = W16 ? add_halves(word[q], local) : local + word[q];
    }
  }
  const uint32_t before = block_exclusive_scan<NT>(local, sm.s_wave, nw_act);
  // Counts in descending bucket order: for W16 the high half (odd bucket) first.
  auto count_at = [&](int q, int h) -> uint32_t {   // h = 0: higher bucket of the word
    if constexpr (W16) return h == 0 ? word[q] >> 16 : word[q] & 0xFFFFu;
    else return word[q];
  };
  // After the scan every thread knows how its buckets stand against t (the
  // bucket holding the K-th largest key) without knowing t: all at or above it
  // (its run ends before K keys), holding it (the finder), or all below. Rows
  // of at most K keys take every bucket (t = 0).
  const bool whole = n <= K;
  const bool above = act && (whole || before + local < (uint32_t)K);
  const bool finder = act && !whole && before < (uint32_t)K && (uint32_t)K <= before + local;
  // The largest count at or above t (a longer segment sends the row to the
  // radix path: it would exceed buf, or make ranking quadratic).
  uint32_t big = 0;
  if (finder) {
    // The word holding bucket t is the first whose running total reaches K:
    // one pass over the words, selecting without branches; the largest count
    // of the words before it folds in on the way (every bucket there is > t).
    uint32_t cum = before, sel_w = 0, sel_cum = 0, mx = 0;
    int sel_q = 0;
    bool found = false;
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      const uint32_t nxt = W16 ? add_halves(word[q], cum) : cum + word[q];
      const bool take = !found && (uint32_t)K <= nxt;
      sel_w = take ? word[q] : sel_w;
      sel_cum = take ? cum : sel_cum;
      sel_q = take ? q : sel_q;
      if constexpr (W16) {
        const uint32_t wm = found || take ? 0u : word[q];
        mx = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(
            __builtin_bit_cast(u16x2_t, mx), __builtin_bit_cast(u16x2_t, wm)));
      } else {
        mx = found || take ? mx : max(mx, word[q]);
      }
      found = found || take;
      cum = nxt;
    }
    int tb;
    uint32_t t_cum, t_cnt;
    if constexpr (W16) {
      const uint32_t c_hi = sel_w >> 16, c_lo = sel_w & 0xFFFFu;
      const bool in_hi = (uint32_t)K <= sel_cum + c_hi;   // t is the word's higher bucket
      tb = nb - 1 - (tid * BPT + BPW * sel_q + (in_hi ? 0 : 1));
      t_cum = in_hi ? sel_cum : sel_cum + c_hi;
      t_cnt = in_hi ? c_hi : c_lo;
      big = max(max(mx >> 16, mx & 0xFFFFu), max(c_hi, in_hi ? 0u : c_lo));
    } else {
      tb = nb - 1 - (tid * BPT + sel_q);
      t_cum = sel_cum;
      t_cnt = sel_w;
      big = max(mx, sel_w);
    }
    sm.s_sel[0] = (uint32_t)tb;
    sm.s_sel[3] = t_cum + t_cnt;   // keys in buckets >= t
  } else if (above) {
    // two 16-bit fields at a time
    if constexpr (W16) {
      uint32_t mx = word[0];
#pragma unroll
      for (int q = 1; q < WPT; ++q) mx = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(
          __builtin_bit_cast(u16x2_t, mx), __builtin_bit_cast(u16x2_t, word[q])));
      big = max(mx >> 16, mx & 0xFFFFu);
    } else {
#pragma unroll
      for (int q = 0; q < WPT; ++q) big = max(big, word[q]);
    }
  }
  if (whole && tid == 0) {
    sm.s_sel[0] = 0u;
    sm.s_sel[3] = (uint32_t)n;
  }
  // Counts become exclusive offsets from the top bucket, in units of U (bytes
  // of buf where they fit 16 bits), for the threads whose buckets reach t.
  // Only buckets >= t are used: their offsets stay below (K + kSegMax) * U and
  // the higher bucket of such a word holds at most kSegMax keys, so the low
  // field's sum cannot carry into the high one; in words wholly below t it may.
  if (above || finder) {
    uint32_t cum = before * U;
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      if constexpr (W16) {
        // (cum, cum + c_hi * U) in the (high, low) fields
        cnt.word(w_top - q) = ((cum << 16) | cum) + (word[q] >> 16) * U;
        cum = __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2_t, word[q]), u16x2_t{U, U}, cum, false);
      } else {
        cnt.word(w_top - q) = cum;
        cum += count_at(q, 0) * U;
      }
    }
  }
  if (big > (uint32_t)kSegMax) atomicMax(&sm.s_sel[2], big);
  __syncthreads();
  if (sm.s_sel[2] != 0u) return false;
  const int t = (int)sm.s_sel[0];
  const uint32_t ncand = sm.s_sel[3];
  // Zero composites past the candidates (the counting sort writes [0, ncand)).
  for (int e = tid; e < kBufPad; e += NT) sm.buf[ncand + e] = 0ull;

  // (65535-4*tid) << 16: key j = 4*tid + c of this thread has low word
  // rjt - (c << 16) + b, one three-operand add (the empty asm keeps the base
  // in a register instead of being recomputed for every key).
  uint32_t rjt = (kIdxMask - 4u * (uint32_t)tid) << 16;
  asm volatile("" : "+v"(rjt));
  // Counting sort of the keys of buckets >= t into their bucket segments.
  // Afterwards bucket b's segment is [end(b+1), end(b)) (end(nb) = 0: the zero
  // word past the buckets). The four atomics of a group are all issued before
  // their results are read.
  row.each4([&](const float (&x)[4], int j0, auto rng) {
    const uint32_t rjs0 = rjt - (((uint32_t)j0 - 4u * (uint32_t)tid) << 16);
    int b[4];
    bool c[4];
    uint32_t raw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      b[e] = bucket(x[e]);
      c[e] = rng.ok(e) && b[e] >= t;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c[e]) raw[e] = cnt.template fetch_add_raw<U>(b[e]);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c[e]) {
        const uint32_t pos = cnt.field(raw[e], b[e]);
        if constexpr (W16)
          at(pos) = bucket_composite(x[e], b[e], rjs0 - ((uint32_t)e << 16));
        else
          at(pos) = composite(x[e], j0 + e);
      }
  });
  __syncthreads();

  // Output records of k slots: stores at slot k or past it are dropped.
  const bool direct = out.gather == nullptr;   // uniform
  const auto ridx = __builtin_amdgcn_make_buffer_rsrc(out.idx, (short)0, K * 4, kRsrcWord3);
  const auto rval = __builtin_amdgcn_make_buffer_rsrc(out.val, (short)0, out.val ? K * 4 : 0, kRsrcWord3);
  // Rank every grouped key inside its segment and store it at its sorted
  // position. NB candidates per thread are ranked together: in a whole batch
  // a wave takes 256 consecutive slots, lane l slots l + 64u (so a wave's
  // loop, which runs to its longest segment, stays in one region of the
  // buffer); in a remainder batch slot p0 is thread p0 - base's;
  // each step reads two consecutive slots of each segment. Slots past a
  // segment's end hold smaller composites (later segments, or the zero pad),
  // so they never count and need no mask. FULL: every slot is < ncand.
  auto rank_batch = [&](uint32_t p0, auto nb_tag, auto full_tag) {
    constexpr int NB = decltype(nb_tag)::value;
    constexpr bool FULL = decltype(full_tag)::value;
    unsigned long long me[NB];
    uint32_t s0[NB], s1[NB], rank[NB];
    int bk[NB];
    uint32_t len = 0;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const uint32_t p = p0 + u * (NB > 1 ? 64u : (uint32_t)NT);
      me[u] = sm.buf[FULL || p < ncand ? p : 0];
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if constexpr (W16) bk[u] = bucket_of(me[u]);
      else bk[u] = bucket(from_ord((uint32_t)(me[u] >> 32)));
      cnt.get_pair(bk[u], s0[u], s1[u]);
    }
    // rank[u] starts at the segment's first slot, so it ends as the sorted slot
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if (!FULL && p0 + u * (NB > 1 ? 64u : (uint32_t)NT) >= ncand) s1[u] = s0[u];
      rank[u] = s0[u] / U;
      len = max(len, s1[u] - s0[u]);
    }
    const unsigned long long* seg[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) seg[u] = &at(s0[u]);
    auto rank_step = [&]() {
      unsigned long long v[NB][2];
#pragma unroll
      for (int u = 0; u < NB; ++u)
#pragma unroll
        for (int w = 0; w < 2; ++w) v[u][w] = seg[u][w];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        seg[u] += 2;
#pragma unroll
        for (int w = 0; w < 2; ++w) rank[u] += v[u][w] > me[u] ? 1u : 0u;
      }
    };
    if constexpr (FULL) {
      // every slot holds a candidate, whose segment holds at least itself
      uint32_t i = 0;
      do rank_step();
      while ((i += 2 * U) < len);
    } else {
      for (uint32_t i = 0; i < len; i += 2 * U) rank_step();
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      // Buckets above t end at or before the K-th slot; bucket t's segment
      // starts below it, so "slot < K" keeps exactly its first need keys.
      const uint32_t slot = rank[u];
      if constexpr (W16) {
        if (direct) {
          if (FULL || s0[u] < s1[u]) out.put_rj(ridx, rval, slot, (uint32_t)me[u], me[u]);
        } else if ((FULL || s0[u] < s1[u]) && slot < (uint32_t)K) {
          out.put_key(slot, bucket_index_of(me[u]), me[u]);
        }
      } else if ((FULL || s0[u] < s1[u]) && slot < (uint32_t)K) {
        out.put(slot, me[u]);
      }
    }
  };
  // Whole batches of four slots per thread, then the rest one slot per thread
  // (the candidate count is often just over a multiple of 4 * NT), skipping
  // waves that hold no candidate.
  using std::integral_constant;
  uint32_t base = 0;
  for (; base + 4 * NT <= ncand; base += 4 * NT)
    rank_batch(base + 4 * (tid & ~63) + (tid & 63), integral_constant<int, 4>{}, integral_constant<bool, true>{});
  for (; base < ncand; base += NT)
    if (base + (tid & ~63) < ncand)   // uniform per wave
      rank_batch(base + tid, integral_constant<int, 1>{}, integral_constant<bool, false>{});
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
// one launch) is held to the register budget of six waves per SIMD, i.e. six
// workgroups per CU (80 VGPRs; its LDS, about 25 KB, fits six in 160 KB; only
// the radix fallback spills a few registers), and the 512-thread kernel (rows
// of 8K-16K keys) to the same six waves, three workgroups per CU (it would
// otherwise take 107 VGPRs and run two: 13% slower on a 16-sequence fp8
// prefill). Explicit attributes: a launch bound's minimum block count did not
// cap the 512-thread kernel's registers.
template <int NT, int R, bool RES, bool KEPT, bool W16, int KMAX>
__global__ __attribute__((amdgpu_flat_work_group_size(1, NT),
                          amdgpu_waves_per_eu(KMAX == kMaxKSmall &&
                                                      (NT == 256 || (NT == 512 && !KEPT))
                                                  ? 6
                                                  : 1)))
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
  for (int w = threadIdx.x; w < (int)(sizeof(sm.cnt) / 16); w += NT)
    reinterpret_cast<uint4*>(sm.cnt)[w] = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x == 0) sm.s_sel[2] = 0u;
  float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
  row.minmax(lo, hi);
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
