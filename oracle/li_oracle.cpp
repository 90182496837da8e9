// Plain fp64 CPU oracle of the LightningIndexer forward pass, in C++17.
//
// TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the CPU
// baseline of the benchmark load it; the product path never does. It shares no
// code with the HIP library (no headers, decoders, tables or helpers) and reads
// nothing but the raw host arrays it is given.
//
// What it computes (the MindSpore "mindspore.ops.lightning_indexer" page,
// formula block; the VllmQuantLightningIndexer README, function description,
// for fp8 / int8 codes with per-token-head dequant scales):
//
//     s_j = sum_g W[g] * ReLU(Q[g] . K[j])                      (f16 / bf16)
//     s_j = sum_g W[g] * ReLU(Sq[g] * Sk[j] * (Qc[g] . Kc[j]))  (e4m3fn / int8)
//
// for every query row and every visible key j, then the k keys of largest
// score, ordered by (score descending, key index ascending). The steps follow
// the TileLang guide's golden (dot products per head, ReLU, weight, sum over
// heads, top-k largest first and sorted), one row at a time, in double. The
// readings where the pages are silent are those of the Python oracle beside
// this file (li_oracle.py): lengths from seqused_* where given (the
// LightningIndexerV2 guide's TND padding for queries), the right-down causal
// rule j <= i + S_k - S_q on actual lengths, compressed keys visible once their
// last original token is, key blocks scored by their largest visible key, the
// first init_num and last local_num blocks always kept (ascending, first), -1 /
// -inf in unused slots, output_idx_offset added to valid indices only.
//
// Rows are dealt round-robin to one std::thread per host core (or the count
// given). The C ABI below takes plain host pointers.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

extern "C" {

// layouts: 0 BSND, 1 TND, 2 PA_BSND; dtypes: 0 f16, 1 bf16, 2 f32, 3 e4m3fn, 4 i8
struct liref_problem {
  int32_t layout_q, layout_k, dtype_qk, dtype_w;
  int32_t batch, s1, s2, n1, n2, d;
  int64_t t1, t2;
  int32_t block_size, max_blocks;
  int32_t sparse_count, sparse_mode, cmp_ratio, block_len, init_num, local_num;
};

// Host arrays, in the shapes of the MindSpore page's parameter list (q (B,S1,N1,D)
// or (T1,N1,D); k (B,S2,N2,D), (T2,N2,D) or (blocks, block_size, N2, D); w and
// q_scale shaped like q without D; k_scale like k without D). Optional ones are NULL.
struct liref_inputs {
  const void* q;
  const void* k;
  const void* w;
  const float* q_scale;
  const float* k_scale;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  const int32_t* seqused_q;
  const int32_t* seqused_k;
  const int32_t* block_table;
  const int32_t* cmp_residual_k;
  const int32_t* output_idx_offset;
};

}  // extern "C"

namespace {

// ---- decoders, from the IEEE 754 / OCP 8-bit field definitions ----
double dec_f16(uint16_t b) {
  const int s = b >> 15, e = (b >> 10) & 0x1F, f = b & 0x3FF;
  double m;
  if (e == 0) m = std::ldexp((double)f, -24);
  else if (e == 31) m = f ? NAN : INFINITY;
  else m = std::ldexp(1024.0 + f, e - 25);
  return s ? -m : m;
}
double dec_bf16(uint16_t b) {
  const int s = b >> 15, e = (b >> 7) & 0xFF, f = b & 0x7F;
  double m;
  if (e == 0) m = std::ldexp((double)f, -133);
  else if (e == 255) m = f ? NAN : INFINITY;
  else m = std::ldexp(128.0 + f, e - 134);
  return s ? -m : m;
}
double dec_e4m3fn(uint8_t b) {
  const int s = b >> 7, e = (b >> 3) & 0xF, f = b & 0x7;
  double m;
  if (e == 0) m = std::ldexp((double)f, -9);
  else if (e == 15 && f == 7) m = NAN;
  else m = std::ldexp(8.0 + f, e - 10);
  return s ? -m : m;
}
double decode(const void* base, int dtype, int64_t i) {
  switch (dtype) {
    case 0: return dec_f16(static_cast<const uint16_t*>(base)[i]);
    case 1: return dec_bf16(static_cast<const uint16_t*>(base)[i]);
    case 2: return (double)static_cast<const float*>(base)[i];
    case 3: return dec_e4m3fn(static_cast<const uint8_t*>(base)[i]);
    default: return (double)static_cast<const int8_t*>(base)[i];
  }
}

int64_t floor_div(int64_t a, int64_t b) {
  const int64_t q = a / b;
  return (a % b != 0 && ((a < 0) != (b < 0))) ? q - 1 : q;
}

struct Oracle {
  const liref_problem& p;
  const liref_inputs& in;

  bool quant() const { return p.dtype_qk == 3 || p.dtype_qk == 4; }

  // Actual (S_q, S_k) of batch b.
  void lengths(int b, int64_t& sq, int64_t& sk) const {
    if (in.seqused_q) sq = in.seqused_q[b];
    else if (p.layout_q == 1) sq = (int64_t)in.cu_seqlens_q[b + 1] - in.cu_seqlens_q[b];
    else sq = p.s1;
    if (in.seqused_k) sk = in.seqused_k[b];
    else if (p.layout_k == 1) sk = (int64_t)in.cu_seqlens_k[b + 1] - in.cu_seqlens_k[b];
    else sk = p.s2;
  }

  int64_t visible(int64_t i, int64_t sq, int64_t sk, int b) const {
    if (i >= sq) return 0;
    if (p.sparse_mode == 0) return sk;
    const int64_t r = p.cmp_ratio > 1 ? p.cmp_ratio : 1;
    const int64_t res = (r > 1 && in.cmp_residual_k) ? in.cmp_residual_k[b] : 0;
    const int64_t v = floor_div(i + 1 + sk * r + res - sq, r);
    return std::max<int64_t>(0, std::min<int64_t>(sk, v));
  }

  // Element index of q / w / q_scale for query position i of batch b, head g.
  int64_t qrow(int b, int64_t i) const {
    return p.layout_q == 1 ? (int64_t)in.cu_seqlens_q[b] + i : (int64_t)b * p.s1 + i;
  }
  // Element index (without D) of key j of batch b, KV head h.
  int64_t krow(int b, int64_t j, int h) const {
    int64_t r;
    if (p.layout_k == 1) r = (int64_t)in.cu_seqlens_k[b] + j;
    else if (p.layout_k == 0) r = (int64_t)b * p.s2 + j;
    else {
      const int64_t blk = in.block_table[(int64_t)b * p.max_blocks + j / p.block_size];
      r = blk * p.block_size + j % p.block_size;
    }
    return r * p.n2 + h;
  }

  // One output row: (b, i) into idx / val (n2 * k each).
  void row(int b, int64_t i, int32_t* idx, float* val) const {
    const int K = p.sparse_count;
    for (int e = 0; e < p.n2 * K; ++e) {
      idx[e] = -1;
      val[e] = -INFINITY;
    }
    int64_t sq, sk;
    lengths(b, sq, sk);
    const int64_t n = visible(i, sq, sk, b);
    if (n == 0) return;
    const int G = p.n1 / p.n2, D = p.d;
    const int64_t qr = qrow(b, i);
    const int32_t off = in.output_idx_offset ? in.output_idx_offset[b] : 0;
    std::vector<double> q((size_t)G * D), w(G), qs(G), kv(D), s(n);
    for (int h = 0; h < p.n2; ++h) {
      for (int g = 0; g < G; ++g) {
        const int64_t hq = qr * p.n1 + h * G + g;
        w[g] = decode(in.w, p.dtype_w, hq);
        qs[g] = quant() ? (double)in.q_scale[hq] : 1.0;
        for (int d = 0; d < D; ++d) q[(size_t)g * D + d] = decode(in.q, p.dtype_qk, hq * D + d);
      }
      // Scores of the visible keys.
      for (int64_t j = 0; j < n; ++j) {
        const int64_t kr = krow(b, j, h);
        for (int d = 0; d < D; ++d) kv[d] = decode(in.k, p.dtype_qk, kr * D + d);
        const double ks = quant() ? (double)in.k_scale[kr] : 1.0;
        double acc = 0.0;
        for (int g = 0; g < G; ++g) {
          double dot = 0.0;
          for (int d = 0; d < D; ++d) dot += q[(size_t)g * D + d] * kv[d];
          double x = quant() ? (qs[g] * ks) * dot : dot;
          acc += w[g] * (x > 0.0 ? x : 0.0);
        }
        s[j] = acc;
      }
      // Key blocks: the largest score over each block's visible keys.
      const int64_t L = p.block_len > 1 ? p.block_len : 1;
      std::vector<double> sb;
      const std::vector<double>* sc = &s;
      if (L > 1) {
        const int64_t nb = (n + L - 1) / L;
        sb.assign(nb, -INFINITY);
        for (int64_t j = 0; j < n; ++j) sb[j / L] = std::max(sb[j / L], s[j]);
        sc = &sb;
      }
      const int64_t nb = (int64_t)sc->size();
      // Blocks always kept: the first init_num and the last local_num.
      std::vector<char> keep(nb, 0);
      for (int64_t c = 0; c < std::min<int64_t>(p.init_num, nb); ++c) keep[c] = 1;
      for (int64_t c = std::max<int64_t>(0, nb - p.local_num); c < nb; ++c) keep[c] = 1;
      std::vector<int64_t> out, rest;
      for (int64_t c = 0; c < nb; ++c) (keep[c] ? out : rest).push_back(c);
      const int64_t room = std::max<int64_t>(0, K - (int64_t)out.size());
      const int64_t take = std::min<int64_t>(room, (int64_t)rest.size());
      std::partial_sort(rest.begin(), rest.begin() + take, rest.end(),
                        [&](int64_t a, int64_t c) {
                          if ((*sc)[a] != (*sc)[c]) return (*sc)[a] > (*sc)[c];
                          return a < c;
                        });
      out.insert(out.end(), rest.begin(), rest.begin() + take);
      for (size_t e = 0; e < out.size() && (int64_t)e < K; ++e) {
        idx[h * K + e] = (int32_t)(out[e] + off);
        val[h * K + e] = (float)(*sc)[out[e]];
      }
    }
  }
};

}  // namespace

extern "C" {

// Output rows of the problem: B*S1 for BSND queries, T1 for TND.
int64_t liref_num_rows(const liref_problem* p) {
  return p->layout_q == 1 ? p->t1 : (int64_t)p->batch * p->s1;
}

// Runs the oracle on `nrows` rows given as (batch, position) pairs in `rows`
// (rows == NULL: every row in order, nrows ignored), writing (rows, n2, k)
// int32 indices and float32 values. nthreads <= 0: one thread per host core.
// Returns the number of threads used, or -1 on a malformed request.
int liref_run(const liref_problem* p, const liref_inputs* in, const int32_t* rows, int64_t nrows,
              int32_t* out_idx, float* out_val, int nthreads) {
  if (!p || !in || !out_idx || !out_val || p->n2 <= 0 || p->n1 % p->n2 != 0) return -1;
  std::vector<int32_t> all;
  if (!rows) {
    for (int b = 0; b < p->batch; ++b) {
      const int64_t nb = p->layout_q == 1 ? (int64_t)in->cu_seqlens_q[b + 1] - in->cu_seqlens_q[b]
                                         : p->s1;
      for (int64_t i = 0; i < nb; ++i) {
        all.push_back(b);
        all.push_back((int32_t)i);
      }
    }
    rows = all.data();
    nrows = (int64_t)all.size() / 2;
  }
  int T = nthreads > 0 ? nthreads : (int)std::thread::hardware_concurrency();
  if (T <= 0) T = 1;
  T = (int)std::min<int64_t>(T, std::max<int64_t>(1, nrows));
  const Oracle o{*p, *in};
  const int64_t stride = (int64_t)p->n2 * p->sparse_count;
  std::vector<std::thread> pool;
  for (int t = 0; t < T; ++t)
    pool.emplace_back([&, t] {
      for (int64_t r = t; r < nrows; r += T)
        o.row(rows[2 * r], rows[2 * r + 1], out_idx + r * stride, out_val + r * stride);
    });
  for (auto& th : pool) th.join();
  return T;
}

}  // extern "C"
