// Host side of the C ABI declared in include/li.h: argument checks, the
// metadata (task table) pass, workspace sizing and kernel launches.
//
// The argument rules follow the checker lists of the CANN LightningIndexerV2
// guide ("约束说明" and "参数校验规则详解": empty tensors rejected, layout pairing,
// cu_seqlens monotone from 0, paged block size, q/k dtype equality), the
// MindSpore page's parameter list (sparse_count range, sparse_mode values,
// pre/next tokens default only, N2 = 1) and the quantised README's constraint
// list (block_table covers the longest sequence, block size multiple of 16 up
// to 1024).
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "li_internal.h"

namespace li {
namespace {

thread_local std::string g_last_error;

li_status vfail(li_status st, const char* fmt, va_list ap) {
  char buf[512];
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  g_last_error = buf;
  return st;
}

li_status fail(li_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(st, fmt, ap);
  va_end(ap);
  return st;
}

#define LI_CHECK(cond, st, ...)            \
  do {                                     \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

constexpr int64_t kInt64Max = 0x7FFFFFFFFFFFFFFFll;

bool is_quant(int dt) { return dt == LI_DTYPE_E4M3FN || dt == LI_DTYPE_I8; }

int64_t elem_bytes(int dt) {
  switch (dt) {
    case LI_DTYPE_F16:
    case LI_DTYPE_BF16: return 2;
    case LI_DTYPE_F32: return 4;
    case LI_DTYPE_E4M3FN:
    case LI_DTYPE_I8: return 1;
    default: return 0;
  }
}

// Checks that depend only on the problem description.
li_status check_problem(const li_problem* p) {
  LI_CHECK(p != nullptr, LI_ERR_INVALID_ARGUMENT, "problem is NULL");
  LI_CHECK(p->api_version == LI_API_VERSION, LI_ERR_INVALID_ARGUMENT,
           "api_version %u, library speaks %d", p->api_version, LI_API_VERSION);
  for (int r : p->reserved) LI_CHECK(r == 0, LI_ERR_INVALID_ARGUMENT, "reserved fields must be zero");
  LI_CHECK(p->layout_q == LI_LAYOUT_BSND || p->layout_q == LI_LAYOUT_TND, LI_ERR_INVALID_ARGUMENT,
           "layout_q must be BSND or TND");
  LI_CHECK(p->layout_k == LI_LAYOUT_BSND || p->layout_k == LI_LAYOUT_TND ||
               p->layout_k == LI_LAYOUT_PA_BSND,
           LI_ERR_INVALID_ARGUMENT, "layout_k must be BSND, TND or PA_BSND");
  LI_CHECK(p->layout_k == LI_LAYOUT_PA_BSND || p->layout_k == p->layout_q, LI_ERR_INVALID_ARGUMENT,
           "layout_k must equal layout_q unless it is PA_BSND");
  LI_CHECK(p->dtype_qk == LI_DTYPE_F16 || p->dtype_qk == LI_DTYPE_BF16 ||
               p->dtype_qk == LI_DTYPE_E4M3FN || p->dtype_qk == LI_DTYPE_I8,
           LI_ERR_INVALID_ARGUMENT, "dtype_qk must be F16, BF16, E4M3FN or I8");
  LI_CHECK(p->dtype_w == LI_DTYPE_F16 || p->dtype_w == LI_DTYPE_BF16 || p->dtype_w == LI_DTYPE_F32,
           LI_ERR_INVALID_ARGUMENT, "dtype_w must be F16, BF16 or F32");
  if (is_quant(p->dtype_qk))
    LI_CHECK(p->dtype_scale == LI_DTYPE_F32, LI_ERR_UNSUPPORTED, "dequant scales must be F32");
  LI_CHECK(p->batch >= 0 && p->n1 >= 0 && p->n2 >= 0 && p->d >= 0, LI_ERR_INVALID_ARGUMENT,
           "negative dimension");
  LI_CHECK(p->batch > 0 && p->n1 > 0 && p->n2 > 0 && p->d > 0, LI_ERR_EMPTY_TENSOR,
           "empty tensor: batch, n1, n2 and d must be positive");
  if (p->layout_q == LI_LAYOUT_BSND) {
    LI_CHECK(p->s1 >= 0, LI_ERR_INVALID_ARGUMENT, "negative s1");
    LI_CHECK(p->s1 > 0, LI_ERR_EMPTY_TENSOR, "empty tensor: s1 is 0");
  } else {
    LI_CHECK(p->t1 >= 0, LI_ERR_INVALID_ARGUMENT, "negative t1");
    LI_CHECK(p->t1 > 0, LI_ERR_EMPTY_TENSOR, "empty tensor: t1 is 0");
    LI_CHECK(p->t1 < (int64_t)1 << 31, LI_ERR_UNSUPPORTED, "t1 must be below 2^31");
  }
  if (p->layout_k == LI_LAYOUT_BSND) {
    LI_CHECK(p->s2 >= 0, LI_ERR_INVALID_ARGUMENT, "negative s2");
    LI_CHECK(p->s2 > 0, LI_ERR_EMPTY_TENSOR, "empty tensor: s2 is 0");
  } else if (p->layout_k == LI_LAYOUT_TND) {
    LI_CHECK(p->t2 >= 0, LI_ERR_INVALID_ARGUMENT, "negative t2");
    LI_CHECK(p->t2 > 0, LI_ERR_EMPTY_TENSOR, "empty tensor: t2 is 0");
    LI_CHECK(p->t2 < (int64_t)1 << 31, LI_ERR_UNSUPPORTED, "t2 must be below 2^31");
  } else {
    LI_CHECK(p->block_size >= 16 && p->block_size <= 1024 && p->block_size % 16 == 0,
             LI_ERR_INVALID_ARGUMENT, "block_size must be a multiple of 16 in [16, 1024], got %d",
             p->block_size);
    LI_CHECK(p->num_blocks >= 0 && p->max_blocks_per_seq >= 0, LI_ERR_INVALID_ARGUMENT,
             "negative paged-cache dimension");
    LI_CHECK(p->num_blocks > 0 && p->max_blocks_per_seq > 0, LI_ERR_EMPTY_TENSOR,
             "empty tensor: num_blocks and max_blocks_per_seq must be positive");
    const int64_t dense = (int64_t)p->block_size * p->n2 * p->d;
    LI_CHECK(p->k_block_stride == 0 || p->k_block_stride >= dense, LI_ERR_INVALID_ARGUMENT,
             "k_block_stride %lld is below one block (%lld elements)",
             (long long)p->k_block_stride, (long long)dense);
    LI_CHECK((p->k_block_stride * elem_bytes(p->dtype_qk)) % 16 == 0, LI_ERR_UNSUPPORTED,
             "k_block_stride must keep blocks 16-byte aligned");
  }
  LI_CHECK(p->n2 == 1, LI_ERR_UNSUPPORTED, "only n2 == 1 is supported (got %d)", p->n2);
  LI_CHECK(p->n1 <= 64, LI_ERR_UNSUPPORTED, "n1 must be at most 64 (got %d)", p->n1);
  LI_CHECK(p->d == 64 || p->d == 128, LI_ERR_UNSUPPORTED, "d must be 64 or 128 (got %d)", p->d);
  LI_CHECK(p->sparse_count >= 1 && p->sparse_count <= 8192, LI_ERR_INVALID_ARGUMENT,
           "sparse_count must be in [1, 8192] (got %d)", p->sparse_count);
  LI_CHECK(p->cmp_ratio >= 0 && p->cmp_ratio <= 128, LI_ERR_INVALID_ARGUMENT,
           "cmp_ratio must be in [0, 128] (0 and 1 mean uncompressed keys), got %d", p->cmp_ratio);
  LI_CHECK(p->sparse_mode == 0 || p->sparse_mode == 3, LI_ERR_INVALID_ARGUMENT,
           "sparse_mode must be 0 or 3 (got %d)", p->sparse_mode);
  LI_CHECK(p->block_len == 0 || p->block_len == 1 || p->block_len == 2 || p->block_len == 4 ||
               p->block_len == 8 || p->block_len == 16,
           LI_ERR_INVALID_ARGUMENT, "block_len must be 0, 1, 2, 4, 8 or 16 (got %d)", p->block_len);
  LI_CHECK(p->init_num >= 0 && p->local_num >= 0, LI_ERR_INVALID_ARGUMENT,
           "init_num and local_num must be non-negative");
  LI_CHECK((int64_t)p->init_num + p->local_num <= p->sparse_count, LI_ERR_INVALID_ARGUMENT,
           "init_num + local_num (%d + %d) exceeds sparse_count %d", p->init_num, p->local_num,
           p->sparse_count);
  LI_CHECK(p->pre_tokens == kInt64Max && p->next_tokens == kInt64Max, LI_ERR_UNSUPPORTED,
           "pre_tokens / next_tokens support only their default 2^63-1");
  LI_CHECK(p->return_value == 0 || p->return_value == 1, LI_ERR_INVALID_ARGUMENT,
           "return_value must be 0 or 1");
  return LI_OK;
}

int32_t cmp_ratio_of(const li_problem& p) { return p.cmp_ratio > 1 ? p.cmp_ratio : 1; }
int32_t block_len_of(const li_problem& p) { return p.block_len > 1 ? p.block_len : 1; }

uint64_t problem_hash(const li_problem& p) {
  // FNV-1a over every field that shapes the task table: the work items, the
  // workspace layout, the top-k records (output offsets row * k, the split of
  // long rows, candidate-list sizes) and the kept-block selection.
  const int64_t f[] = {p.layout_q, p.layout_k, p.dtype_qk, p.batch, p.s1, p.s2, p.n1, p.n2, p.d,
                       p.t1, p.t2, p.block_size, p.max_blocks_per_seq, p.num_blocks,
                       p.sparse_mode, cmp_ratio_of(p), block_len_of(p), p.sparse_count,
                       p.init_num, p.local_num};
  uint64_t h = 1469598103934665603ull;
  const unsigned char* b = reinterpret_cast<const unsigned char*>(f);
  for (size_t i = 0; i < sizeof f; ++i) {
    h ^= b[i];
    h *= 1099511628211ull;
  }
  return h;
}

int64_t num_rows(const li_problem& p) {
  return p.layout_q == LI_LAYOUT_BSND ? (int64_t)p.batch * p.s1 : p.t1;
}

li_status check_meta(const li_problem& p, const void* meta_host, const MetaHeader** out) {
  LI_CHECK(meta_host != nullptr, LI_ERR_INVALID_ARGUMENT, "meta_host is NULL");
  const MetaHeader* h = static_cast<const MetaHeader*>(meta_host);
  LI_CHECK(h->magic == kMetaMagic && h->version == kMetaVersion, LI_ERR_METADATA_MISMATCH,
           "meta_host does not hold a task table of this library version");
  LI_CHECK(h->problem_hash == problem_hash(p) && h->batch == p.batch &&
               h->num_rows == num_rows(p),
           LI_ERR_METADATA_MISMATCH, "task table was built for another problem");
  // The fields the row records depend on are also compared one by one, so that
  // a hash collision cannot let a table of another k through.
  LI_CHECK(h->sparse_count == p.sparse_count && h->init_num == p.init_num &&
               h->local_num == p.local_num,
           LI_ERR_METADATA_MISMATCH,
           "task table was built for sparse_count %d, init_num %d, local_num %d (problem: %d, %d, %d)",
           h->sparse_count, h->init_num, h->local_num, p.sparse_count, p.init_num, p.local_num);
  *out = h;
  return LI_OK;
}

template <typename T>
const T* meta_ptr(const void* base, uint64_t off) {
  return reinterpret_cast<const T*>(static_cast<const uint8_t*>(base) + off);
}

}  // namespace

li_status set_error(li_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(st, fmt, ap);
  va_end(ap);
  return st;
}

}  // namespace li

using namespace li;

extern "C" {

int32_t li_api_version(void) { return LI_API_VERSION; }

const char* li_last_error(void) { return g_last_error.c_str(); }

li_status li_metadata(const li_problem* p, const li_lengths* L, int32_t num_cus, void* meta_host,
                      size_t meta_capacity, size_t* meta_bytes) {
  try {
    li_status st = check_problem(p);
    if (st != LI_OK) return st;
    LI_CHECK(L != nullptr, LI_ERR_INVALID_ARGUMENT, "lengths is NULL");
    LI_CHECK(meta_bytes != nullptr, LI_ERR_INVALID_ARGUMENT, "meta_bytes is NULL");
    if (num_cus <= 0) num_cus = 256;
    const int B = p->batch;

    // ---- per-sequence lengths, with the pages' rules ----
    std::vector<int32_t> sq(B), sk(B), rows(B), row_base(B), k_base(B);
    if (p->layout_q == LI_LAYOUT_TND) {
      LI_CHECK(L->cu_seqlens_q != nullptr, LI_ERR_INVALID_ARGUMENT,
               "TND queries need cu_seqlens_q");
      LI_CHECK(L->cu_seqlens_q[0] == 0, LI_ERR_INVALID_ARGUMENT, "cu_seqlens_q[0] must be 0");
      for (int b = 0; b < B; ++b) {
        const int64_t n64 = (int64_t)L->cu_seqlens_q[b + 1] - L->cu_seqlens_q[b];
        LI_CHECK(n64 >= 0 && L->cu_seqlens_q[b] >= 0, LI_ERR_INVALID_ARGUMENT,
                 "cu_seqlens_q must be non-decreasing from 0");
        const int32_t n = (int32_t)n64;
        rows[b] = n;
        row_base[b] = L->cu_seqlens_q[b];
        sq[b] = n;
        if (L->seqused_q) {
          LI_CHECK(L->seqused_q[b] >= 0 && L->seqused_q[b] <= n, LI_ERR_INVALID_ARGUMENT,
                   "seqused_q[%d]=%d exceeds the cu_seqlens_q length %d", b, L->seqused_q[b], n);
          sq[b] = L->seqused_q[b];
        }
      }
      LI_CHECK(L->cu_seqlens_q[B] == p->t1, LI_ERR_INVALID_ARGUMENT,
               "cu_seqlens_q[B]=%d differs from t1=%lld", L->cu_seqlens_q[B], (long long)p->t1);
    } else {
      LI_CHECK(L->cu_seqlens_q == nullptr, LI_ERR_INVALID_ARGUMENT,
               "BSND queries do not take cu_seqlens_q");
      LI_CHECK((int64_t)B * p->s1 < ((int64_t)1 << 31), LI_ERR_UNSUPPORTED,
               "batch * s1 must be below 2^31");
      for (int b = 0; b < B; ++b) {
        rows[b] = p->s1;
        row_base[b] = b * p->s1;
        sq[b] = p->s1;
        if (L->seqused_q) {
          LI_CHECK(L->seqused_q[b] >= 0 && L->seqused_q[b] <= p->s1, LI_ERR_INVALID_ARGUMENT,
                   "seqused_q[%d]=%d outside [0, s1=%d]", b, L->seqused_q[b], p->s1);
          sq[b] = L->seqused_q[b];
        }
      }
    }
    if (p->layout_k == LI_LAYOUT_TND) {
      LI_CHECK(L->cu_seqlens_k != nullptr, LI_ERR_INVALID_ARGUMENT, "TND keys need cu_seqlens_k");
      LI_CHECK(L->cu_seqlens_k[0] == 0, LI_ERR_INVALID_ARGUMENT, "cu_seqlens_k[0] must be 0");
      for (int b = 0; b < B; ++b) {
        const int64_t n64 = (int64_t)L->cu_seqlens_k[b + 1] - L->cu_seqlens_k[b];
        LI_CHECK(n64 >= 0 && L->cu_seqlens_k[b] >= 0, LI_ERR_INVALID_ARGUMENT,
                 "cu_seqlens_k must be non-decreasing from 0");
        const int32_t n = (int32_t)n64;
        k_base[b] = L->cu_seqlens_k[b];
        sk[b] = n;
        if (L->seqused_k) {
          LI_CHECK(L->seqused_k[b] >= 0 && L->seqused_k[b] <= n, LI_ERR_INVALID_ARGUMENT,
                   "seqused_k[%d]=%d exceeds the cu_seqlens_k length %d", b, L->seqused_k[b], n);
          sk[b] = L->seqused_k[b];
        }
      }
      LI_CHECK(L->cu_seqlens_k[B] == p->t2, LI_ERR_INVALID_ARGUMENT,
               "cu_seqlens_k[B]=%d differs from t2=%lld", L->cu_seqlens_k[B], (long long)p->t2);
    } else if (p->layout_k == LI_LAYOUT_BSND) {
      LI_CHECK(L->cu_seqlens_k == nullptr, LI_ERR_INVALID_ARGUMENT,
               "BSND keys do not take cu_seqlens_k");
      LI_CHECK((int64_t)B * p->s2 < ((int64_t)1 << 31), LI_ERR_UNSUPPORTED,
               "batch * s2 must be below 2^31");
      for (int b = 0; b < B; ++b) {
        k_base[b] = b * p->s2;
        sk[b] = p->s2;
        if (L->seqused_k) {
          LI_CHECK(L->seqused_k[b] >= 0 && L->seqused_k[b] <= p->s2, LI_ERR_INVALID_ARGUMENT,
                   "seqused_k[%d]=%d outside [0, s2=%d]", b, L->seqused_k[b], p->s2);
          sk[b] = L->seqused_k[b];
        }
      }
    } else {
      LI_CHECK(L->cu_seqlens_k == nullptr, LI_ERR_INVALID_ARGUMENT,
               "PA_BSND keys do not take cu_seqlens_k");
      LI_CHECK(L->seqused_k != nullptr, LI_ERR_INVALID_ARGUMENT, "PA_BSND keys need seqused_k");
      const int64_t cap = (int64_t)p->max_blocks_per_seq * p->block_size;
      for (int b = 0; b < B; ++b) {
        k_base[b] = 0;
        sk[b] = L->seqused_k[b];
        LI_CHECK(sk[b] >= 0, LI_ERR_INVALID_ARGUMENT, "seqused_k[%d] is negative", b);
        LI_CHECK(sk[b] <= cap, LI_ERR_INVALID_ARGUMENT,
                 "seqused_k[%d]=%d needs more than max_blocks_per_seq=%d blocks", b, sk[b],
                 p->max_blocks_per_seq);
      }
    }

    // ---- compressed keys and index offsets (V2 guide, constraint list) ----
    const int32_t cr = cmp_ratio_of(*p);
    std::vector<int32_t> cres(B, 0), ioff(B, 0);
    if (cr > 1 && p->sparse_mode == 3) {
      LI_CHECK(L->cmp_residual_k != nullptr, LI_ERR_INVALID_ARGUMENT,
               "cmp_ratio > 1 with sparse_mode 3 needs cmp_residual_k");
      for (int b = 0; b < B; ++b) {
        cres[b] = L->cmp_residual_k[b];
        LI_CHECK(cres[b] >= 0 && cres[b] < cr, LI_ERR_INVALID_ARGUMENT,
                 "cmp_residual_k[%d]=%d outside [0, cmp_ratio=%d)", b, cres[b], cr);
        LI_CHECK((int64_t)sk[b] * cr + cres[b] < ((int64_t)1 << 31), LI_ERR_UNSUPPORTED,
                 "sequence %d is longer than 2^31 original tokens", b);
      }
    } else {
      LI_CHECK(L->cmp_residual_k == nullptr, LI_ERR_INVALID_ARGUMENT,
               "cmp_residual_k is taken only with cmp_ratio > 1 and sparse_mode 3");
    }
    if (L->output_idx_offset) {
      for (int b = 0; b < B; ++b) {
        ioff[b] = L->output_idx_offset[b];
        LI_CHECK(ioff[b] >= 0, LI_ERR_INVALID_ARGUMENT, "output_idx_offset[%d]=%d is negative", b,
                 ioff[b]);
        LI_CHECK((int64_t)ioff[b] + (sk[b] > 0 ? sk[b] - 1 : 0) <= 0x7FFFFFFFll,
                 LI_ERR_INVALID_ARGUMENT,
                 "output_idx_offset[%d]=%d pushes key index %d past INT32_MAX", b, ioff[b],
                 sk[b] - 1);
      }
    }
    auto visible = [&](int b, int i) {
      return visible_keys(i, sq[b], sk[b], p->sparse_mode, cr, cres[b]);
    };
    // Rows select over blocks of bl keys when block_len > 1: one stored score
    // per block.
    const int32_t bl = block_len_of(*p);
    auto blocks = [&](int n) { return (n + bl - 1) / bl; };

    // ---- variant and tiling ----
    int max_sq = 0, max_sk = 0;
    for (int b = 0; b < B; ++b) {
      max_sq = std::max(max_sq, sq[b]);
      max_sk = std::max(max_sk, sk[b]);
    }
    const bool quant = p->dtype_qk == LI_DTYPE_E4M3FN || p->dtype_qk == LI_DTYPE_I8;
    const int variant = max_sq <= 2 ? kVarDecode
                        : max_sq <= 4 ? kVarMid
                        : quant ? kVarQuant : kVarPrefill;
    const int TQ = kVariantTileQ[variant];
    const int KT = kVariantTileK[variant];

    int64_t pairs = 0;
    for (int b = 0; b < B; ++b)
      for (int i = 0; i < sq[b]; ++i) pairs += visible(b, i);
    // Each key chunk of a row tile re-reads the tile's query heads, so rows are
    // split along keys only when there are too few row tiles to fill the CUs.
    int64_t tiles = 0;
    for (int b = 0; b < B; ++b) tiles += (sq[b] + TQ - 1) / TQ;
    const int64_t whole = std::max<int64_t>(KT, ((int64_t)max_sk + KT - 1) / KT * KT);
    int64_t chunk = whole;
    if (tiles < 2ll * num_cus) {
      // Four items per CU (eight for decode, whose items are short and run two
      // per CU): fewer leave a tail, more repeat the query loads.
      const int64_t target_items = (variant == kVarDecode ? 8ll : 4ll) * num_cus;
      chunk = (pairs + TQ * target_items - 1) / (TQ * target_items);
      chunk = std::max<int64_t>(chunk, 8ll * KT);
      chunk = std::min<int64_t>((chunk + KT - 1) / KT * KT, whole);
    }

    // ---- sequences ----
    std::vector<BatchRec> recs(B);
    int64_t ws = 0;
    for (int b = 0; b < B; ++b) {
      BatchRec& r = recs[b];
      r.ws_off = ws;
      r.row_base = row_base[b];
      r.k_base = k_base[b];
      r.s_q = sq[b];
      r.s_k = sk[b];
      r.ld = std::max(4, (blocks(sk[b]) + 3) / 4 * 4);
      r.rows = rows[b];
      r.cmp_res = cres[b];
      r.reserved = 0;
      ws += (int64_t)sq[b] * r.ld;
    }

    // ---- work items, heaviest first ----
    struct Cand {
      WorkItem w;
      int64_t cost;
    };
    std::vector<Cand> cands;
    for (int b = 0; b < B; ++b) {
      for (int q0 = 0; q0 < sq[b]; q0 += TQ) {
        const int qe = std::min(q0 + TQ, sq[b]);
        const int nvmax = visible(b, qe - 1);
        for (int64_t k0 = 0; k0 < nvmax; k0 += chunk) {
          const int k1 = (int)std::min<int64_t>(k0 + chunk, nvmax);
          int64_t cost = 0;
          for (int i = q0; i < qe; ++i) {
            const int nv = visible(b, i);
            cost += std::max<int64_t>(0, std::min<int64_t>(nv, k1) - k0);
          }
          cands.push_back({{b, q0, (int)k0, k1}, cost});
        }
      }
    }
    std::stable_sort(cands.begin(), cands.end(),
                     [](const Cand& x, const Cand& y) { return x.cost > y.cost; });
    LI_CHECK(cands.size() < ((size_t)1 << 31), LI_ERR_UNSUPPORTED, "too many work items");

    // ---- top-k records: two passes, each grouped by size class, longest first ----
    const int64_t nrows = num_rows(*p);
    LI_CHECK(nrows < ((int64_t)1 << 31), LI_ERR_UNSUPPORTED, "too many output rows");
    const int32_t K = p->sparse_count;
    // Split long rows only where rows are too few to fill the CUs (a split adds
    // a pass over k candidates per chunk) and never with always-kept blocks.
    const bool may_split = K <= kSplitMaxK && p->init_num == 0 && p->local_num == 0 &&
                           nrows < (int64_t)kSplitRowsPerCu * num_cus;
    // Candidate lists live after the scores: values, then indices.
    const int64_t cand_val_off = (ws + 3) / 4 * 4;
    int64_t cand = 0;   // candidate floats allotted so far (multiple of 4 per split row)
    std::vector<std::vector<RowRec>> pass[2];
    pass[0].resize(kTopkClasses);
    pass[1].resize(kTopkClasses);
    int64_t covered = 0;
    int32_t split_rows = 0;
    for (int b = 0; b < B; ++b) {
      for (int i = 0; i < rows[b]; ++i) {
        const int n = i < sq[b] ? blocks(visible(b, i)) : 0;
        const int64_t off = n > 0 ? recs[b].ws_off + (int64_t)i * recs[b].ld : 0;
        const int32_t row = (int32_t)(row_base[b] + i);
        if (!may_split || n <= kTopkClassKeys[0]) {
          pass[0][topk_class(n)].push_back({off, (int64_t)row * K, n, ioff[b], row, kRowWhole});
          continue;
        }
        // Chunk q covers keys [e_q, e_{q+1}) with e_q = 4*floor(q*n / (4c)):
        // 16-byte aligned starts, lengths within 4 of n/c, so in
        // (kSplitKeys/2 - 4, kSplitKeys + 4] -- above k and inside class 0.
        const int64_t c = ((int64_t)n + kSplitKeys - 1) / kSplitKeys;
        auto edge = [&](int64_t q) { return q >= c ? (int64_t)n : 4 * ((q * n) / (4 * c)); };
        for (int64_t q = 0; q < c; ++q) {
          const int64_t e0 = edge(q), e1 = edge(q + 1);
          pass[0][0].push_back({off + e0, cand + q * K, (int32_t)(e1 - e0), (int32_t)e0, row,
                                kRowChunk});
        }
        const int64_t nc = c * K;
        LI_CHECK(nc < ((int64_t)1 << 31), LI_ERR_UNSUPPORTED, "row %d has too many candidates",
                 row);
        pass[1][topk_class((int)nc)].push_back(
            {cand_val_off + cand, (int64_t)row * K, (int32_t)nc, ioff[b], row, kRowMerge});
        cand += (nc + 3) / 4 * 4;
        ++split_rows;
      }
      covered += rows[b];
    }
    LI_CHECK(covered == nrows, LI_ERR_INVALID_ARGUMENT,
             "sequences cover %lld output rows, the problem has %lld", (long long)covered,
             (long long)nrows);
    // The second pass is short (one record per split row) and runs alone: one
    // launch, in the class of its longest record, instead of one per class.
    for (int c = kTopkClasses - 1; c > 0; --c) {
      if (pass[1][c].empty()) continue;
      for (int d = 0; d < c; ++d) {
        pass[1][c].insert(pass[1][c].end(), pass[1][d].begin(), pass[1][d].end());
        pass[1][d].clear();
      }
      break;
    }
    const int64_t cand_idx_off = cand_val_off + cand;
    if (cand > 0) ws = cand_idx_off + cand;
    int64_t nrecs = 0;
    for (int q = 0; q < 2; ++q)
      for (const auto& v : pass[q]) nrecs += (int64_t)v.size();
    LI_CHECK(nrecs < ((int64_t)1 << 31), LI_ERR_UNSUPPORTED, "too many top-k records");

    const size_t off_b = sizeof(MetaHeader);
    const size_t off_i = off_b + sizeof(BatchRec) * (size_t)B;
    const size_t off_r = off_i + sizeof(WorkItem) * cands.size();
    const size_t need = off_r + sizeof(RowRec) * (size_t)nrecs;
    *meta_bytes = need;
    if (meta_host == nullptr) return LI_OK;
    LI_CHECK(meta_capacity >= need, LI_ERR_BUFFER_TOO_SMALL,
             "meta buffer holds %zu bytes, %zu needed", meta_capacity, need);

    MetaHeader h;
    std::memset(&h, 0, sizeof h);
    h.magic = kMetaMagic;
    h.version = kMetaVersion;
    h.problem_hash = problem_hash(*p);
    h.batch = B;
    h.num_items = (int32_t)cands.size();
    h.num_rows = num_rows(*p);
    h.variant = variant;
    h.tile_q = TQ;
    h.key_chunk = (int32_t)chunk;
    h.num_cus = num_cus;
    h.ws_floats = ws;
    h.visible_pairs = pairs;
    h.off_batches = off_b;
    h.off_items = off_i;
    h.max_sk = max_sk;
    h.max_sq = max_sq;
    h.off_rows = off_r;
    h.split_rows = split_rows;
    h.cand_val_off = cand > 0 ? cand_val_off : 0;
    h.cand_idx_off = cand > 0 ? cand_idx_off : 0;
    h.num_recs = nrecs;
    h.sparse_count = p->sparse_count;
    h.init_num = p->init_num;
    h.local_num = p->local_num;
    uint8_t* dst = static_cast<uint8_t*>(meta_host);
    std::memcpy(dst + off_b, recs.data(), sizeof(BatchRec) * (size_t)B);
    WorkItem* items = reinterpret_cast<WorkItem*>(dst + off_i);
    for (size_t n = 0; n < cands.size(); ++n) items[n] = cands[n].w;
    RowRec* rrecs = reinterpret_cast<RowRec*>(dst + off_r);
    int32_t pos = 0;
    for (int q = 0; q < 2; ++q) {
      for (int c = 0; c < kTopkClasses; ++c) {
        auto& v = pass[q][c];
        std::stable_sort(v.begin(), v.end(),
                         [](const RowRec& x, const RowRec& y) { return x.n > y.n; });
        h.row_class[q * kTopkClasses + c] = pos;
        for (const RowRec& rc : v) rrecs[pos++] = rc;
      }
    }
    h.row_class[2 * kTopkClasses] = pos;
    std::memcpy(dst, &h, sizeof h);
    return LI_OK;
  } catch (const std::exception& e) {
    return fail(LI_ERR_INVALID_ARGUMENT, "li_metadata: %s", e.what());
  } catch (...) {
    return fail(LI_ERR_INVALID_ARGUMENT, "li_metadata: unknown failure");
  }
}

li_status li_workspace_size(const li_problem* p, const void* meta_host, size_t* bytes) {
  li_status st = check_problem(p);
  if (st != LI_OK) return st;
  LI_CHECK(bytes != nullptr, LI_ERR_INVALID_ARGUMENT, "bytes is NULL");
  const MetaHeader* h = nullptr;
  st = check_meta(*p, meta_host, &h);
  if (st != LI_OK) return st;
  *bytes = (size_t)std::max<int64_t>(h->ws_floats, 1) * sizeof(float);
  return LI_OK;
}

li_status li_score(const li_problem* p, const li_inputs* in, const void* meta_host,
                   const void* meta_dev, void* ws, size_t ws_bytes, void* stream) {
  li_status st = check_problem(p);
  if (st != LI_OK) return st;
  const MetaHeader* h = nullptr;
  st = check_meta(*p, meta_host, &h);
  if (st != LI_OK) return st;
  LI_CHECK(in != nullptr, LI_ERR_INVALID_ARGUMENT, "inputs is NULL");
  LI_CHECK(in->q && in->k && in->w, LI_ERR_INVALID_ARGUMENT, "q, k and w are required");
  if (is_quant(p->dtype_qk))
    LI_CHECK(in->q_scale && in->k_scale, LI_ERR_INVALID_ARGUMENT,
             "quantised q/k need q_scale and k_scale");
  if (p->layout_k == LI_LAYOUT_PA_BSND)
    LI_CHECK(in->block_table != nullptr, LI_ERR_INVALID_ARGUMENT, "PA_BSND keys need block_table");
  LI_CHECK(meta_dev != nullptr, LI_ERR_INVALID_ARGUMENT, "meta_dev is NULL");
  LI_CHECK(ws != nullptr, LI_ERR_INVALID_ARGUMENT, "workspace is NULL");
  const size_t need = (size_t)std::max<int64_t>(h->ws_floats, 1) * sizeof(float);
  LI_CHECK(ws_bytes >= need, LI_ERR_WORKSPACE_TOO_SMALL, "workspace holds %zu bytes, %zu needed",
           ws_bytes, need);
  LI_CHECK(((uintptr_t)in->q % 16) == 0 && ((uintptr_t)in->k % 16) == 0, LI_ERR_INVALID_ARGUMENT,
           "q and k must be 16-byte aligned");
  LI_CHECK(((uintptr_t)ws % 16) == 0, LI_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");

  ScoreArgs a;
  a.q = static_cast<const uint8_t*>(in->q);
  a.k = static_cast<const uint8_t*>(in->k);
  a.w = in->w;
  a.q_scale = in->q_scale;
  a.k_scale = in->k_scale;
  a.block_table = in->block_table;
  a.batches = meta_ptr<BatchRec>(meta_dev, h->off_batches);
  a.items = meta_ptr<WorkItem>(meta_dev, h->off_items);
  a.ws = static_cast<float*>(ws);
  a.k_block_stride = p->k_block_stride ? p->k_block_stride
                                       : (int64_t)p->block_size * p->n2 * p->d;
  a.num_blocks = p->num_blocks;
  a.n1 = p->n1;
  a.layout_k = p->layout_k;
  a.dtype_w = p->dtype_w;
  a.block_size = p->block_size;
  a.block_shift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if (p->block_size == (1 << sh)) a.block_shift = sh;
  a.max_blocks = p->max_blocks_per_seq;
  a.sparse_mode = p->sparse_mode;
  a.cmp_ratio = cmp_ratio_of(*p);
  a.key_block = block_len_of(*p);
  a.key_block_shift = 0;
  while ((1 << a.key_block_shift) < a.key_block) ++a.key_block_shift;
  const hipError_t e = launch_score(*p, h->variant, h->num_items, a, (hipStream_t)stream);
  LI_CHECK(e == hipSuccess, LI_ERR_HIP, "score kernel launch: %s", hipGetErrorString(e));
  return LI_OK;
}

li_status li_topk(const li_problem* p, const void* meta_host, const void* meta_dev,
                  void* ws, size_t ws_bytes, int32_t* sparse_indices,
                  float* sparse_values, void* stream) {
  li_status st = check_problem(p);
  if (st != LI_OK) return st;
  const MetaHeader* h = nullptr;
  st = check_meta(*p, meta_host, &h);
  if (st != LI_OK) return st;
  LI_CHECK(meta_dev != nullptr, LI_ERR_INVALID_ARGUMENT, "meta_dev is NULL");
  LI_CHECK(ws != nullptr, LI_ERR_INVALID_ARGUMENT, "workspace is NULL");
  const size_t need = (size_t)std::max<int64_t>(h->ws_floats, 1) * sizeof(float);
  LI_CHECK(ws_bytes >= need, LI_ERR_WORKSPACE_TOO_SMALL, "workspace holds %zu bytes, %zu needed",
           ws_bytes, need);
  LI_CHECK(sparse_indices != nullptr, LI_ERR_INVALID_ARGUMENT, "sparse_indices is NULL");
  LI_CHECK(!p->return_value || sparse_values != nullptr, LI_ERR_INVALID_ARGUMENT,
           "return_value needs sparse_values");
  LI_CHECK(((uintptr_t)ws % 16) == 0, LI_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  TopkArgs a;
  a.ws = static_cast<const float*>(ws);
  a.rows = meta_ptr<RowRec>(meta_dev, h->off_rows);
  a.out_idx = sparse_indices;
  a.out_val = p->return_value ? sparse_values : nullptr;
  a.k = p->sparse_count;
  a.init_num = p->init_num;
  a.local_num = p->local_num;
  a.cand_val_off = h->cand_val_off;
  a.cand_val = h->split_rows > 0 ? static_cast<float*>(ws) + h->cand_val_off : nullptr;
  a.cand_idx = h->split_rows > 0 ? reinterpret_cast<int32_t*>(static_cast<float*>(ws) + h->cand_idx_off)
                                 : nullptr;
  for (int c = 0; c <= 2 * kTopkClasses; ++c) a.row_class[c] = h->row_class[c];
  const hipError_t e = launch_topk(*p, a, (hipStream_t)stream);
  LI_CHECK(e == hipSuccess, LI_ERR_HIP, "top-k kernel launch: %s", hipGetErrorString(e));
  return LI_OK;
}

li_status li_indexer(const li_problem* p, const li_inputs* in, const void* meta_host,
                     const void* meta_dev, void* ws, size_t ws_bytes, int32_t* sparse_indices,
                     float* sparse_values, void* stream) {
  // Validate both halves before enqueueing either.
  li_status st = check_problem(p);
  if (st != LI_OK) return st;
  LI_CHECK(sparse_indices != nullptr, LI_ERR_INVALID_ARGUMENT, "sparse_indices is NULL");
  LI_CHECK(!p->return_value || sparse_values != nullptr, LI_ERR_INVALID_ARGUMENT,
           "return_value needs sparse_values");
  st = li_score(p, in, meta_host, meta_dev, ws, ws_bytes, stream);
  if (st != LI_OK) return st;
  return li_topk(p, meta_host, meta_dev, ws, ws_bytes, sparse_indices, sparse_values, stream);
}

}  // extern "C"
