// Internal definitions shared by the host side of the library and its kernels:
// the metadata (task table) layout, score-kernel variants, kernel arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/li.h"

namespace li {

// ---------------------------------------------------------------------------
// Task table written by li_metadata (host), read by the kernels (device).
//
//   [MetaHeader][BatchRec x batch][WorkItem x num_items][RowRec x num_recs]
//
// Each BatchRec describes one sequence; each WorkItem is one workgroup of the
// score kernel: query rows [q0, q0 + tile_q) of sequence b against keys
// [k0, k1). Items are sorted by descending visible-pair count. Each RowRec is
// one top-k workgroup: it carries the visible-key count, the workspace offset
// of the scores and where the result goes, so that the workgroup needs one
// record. Records run in two passes, each grouped by size class and, inside a
// class, longest first. Normally every output row is one record of the first
// pass. When a problem has few rows (fewer than two per CU) and k <= 2048, a
// row of more than kSplitKeys keys is split instead: each of its chunks (at
// most kSplitKeys keys, more than k) is a first-pass record that writes its
// sorted top k (indices and values) to a candidate list in the workspace, and
// a second-pass record selects the row's top k among the chunk lists.
// ---------------------------------------------------------------------------
constexpr uint32_t kMetaMagic = 0x444D494Cu;  // "LIMD"
constexpr uint32_t kMetaVersion = 8;

// Top-k size classes: class c holds the rows of at most kTopkClassKeys[c]
// visible keys (the last class is unbounded) and runs with kTopkClassThreads[c]
// threads per row.
constexpr int kTopkClasses = 4;
constexpr int kTopkClassKeys[kTopkClasses] = {8192, 16384, 32768, 0x7FFFFFFF};
constexpr int kTopkClassThreads[kTopkClasses] = {256, 512, 1024, 1024};
inline int topk_class(int n) {
  int c = 0;
  while (c + 1 < kTopkClasses && n > kTopkClassKeys[c]) ++c;
  return c;
}

// Row splitting: chunk length bound (a multiple-of-4 split of a row into
// ceil(n / kSplitKeys) chunks keeps every chunk within the first class), the
// largest k it is used for, and the row count below which (per CU) it is used.
constexpr int kSplitKeys = 8188;
constexpr int kSplitMaxK = 2048;
constexpr int kSplitRowsPerCu = 2;

struct MetaHeader {
  uint32_t magic;
  uint32_t version;
  uint64_t problem_hash;   // hash of the li_problem fields that shape the work
  int32_t batch;
  int32_t num_items;
  int64_t num_rows;        // output rows: B*S1 (BSND) or T1 (TND)
  int32_t variant;         // score-kernel variant (ScoreVariant)
  int32_t tile_q;          // query rows per work item
  int32_t key_chunk;       // keys per work item (upper bound)
  int32_t num_cus;
  int64_t ws_floats;       // workspace size in floats
  int64_t visible_pairs;   // sum over rows of visible keys
  uint64_t off_batches;    // byte offset of the BatchRec array
  uint64_t off_items;      // byte offset of the WorkItem array
  int32_t max_sk;
  int32_t max_sq;
  uint64_t off_rows;       // byte offset of the RowRec array
  // First RowRec of each class of each pass: pass q, class c starts at
  // row_class[q * kTopkClasses + c]; row_class[2 * kTopkClasses] = num_recs.
  int32_t row_class[2 * kTopkClasses + 1];
  int32_t split_rows;      // output rows handled by chunks + a second-pass record
  int64_t cand_val_off;    // workspace float offset of the candidate values
  int64_t cand_idx_off;    // ... of the candidate indices (int32 in float slots)
  int64_t num_recs;        // RowRec records of both passes
  // Selection fields the row records are laid out for (output offsets row*k,
  // the split decision, candidate-list sizes); also covered by problem_hash.
  int32_t sparse_count;
  int32_t init_num;
  int32_t local_num;
  int32_t reserved;
};
static_assert(sizeof(MetaHeader) == 176, "header size");

struct BatchRec {
  int64_t ws_off;   // first workspace float of the sequence
  int32_t row_base; // first output row == first q / w row of the sequence
  int32_t k_base;   // first key row (TND: cu_seqlens_k[b]; BSND: b*S2; PA: 0)
  int32_t s_q;      // actual query length
  int32_t s_k;      // actual key length (compressed keys when cmp_ratio > 1)
  int32_t ld;       // workspace row stride in floats (multiple of 4)
  int32_t rows;     // output rows allotted to the sequence (S1 for BSND, the cu_seqlens_q length for TND)
  int32_t cmp_res;  // original tokens past the last whole compressed key (0 if none)
  int32_t reserved;
};
static_assert(sizeof(BatchRec) == 40, "batch record size");

struct WorkItem {
  int32_t b, q0, k0, k1;
};
static_assert(sizeof(WorkItem) == 16, "work item size");

// What a top-k record selects from and where its result goes.
enum RowKind : int32_t {
  kRowWhole = 0,  // an output row: scores -> output row
  kRowChunk = 1,  // a chunk of a split row: scores -> candidate list (indices and values)
  kRowMerge = 2,  // a split row: its chunks' candidate lists -> output row
};

struct RowRec {
  int64_t ws_off;      // first workspace float of the scores (kRowMerge: candidate values)
  int64_t out_off;     // first output element: row * k in the outputs, or (kRowChunk)
                       // the candidate-list offset from cand_val_off / cand_idx_off
  int32_t n;           // keys to select from: visible keys (or key blocks when
                       // block_len > 1; 0 for rows past a sequence's actual
                       // length), a chunk's keys, or a split row's candidates
  int32_t idx_offset;  // added to every returned index: output_idx_offset, or
                       // (kRowChunk) the chunk's first key
  int32_t row;         // output row (B*S1 rows for BSND, T1 for TND)
  int32_t kind;        // RowKind
};
static_assert(sizeof(RowRec) == 32, "row record size");

// Score-kernel variants: waves of one query row each, arranged as WQ rows x WK
// key slices; KT keys staged in LDS per step. Prefill workgroups have 8 waves
// (one per CU); the short-sequence ones have 4 and run two per CU, so that one
// workgroup's start (query loads, first stages) overlaps the other's key loop.
// fp8 / int8 prefill has 4 waves in each of three workgroups per CU (three
// waves per SIMD: its epilogue, not the matrix cores, bounds it, and the third
// wave hides the epilogue's wait for the MFMA results).
enum ScoreVariant : int32_t {
  kVarPrefill = 0,  // WQ=8, WK=1: 8 query rows share each staged key tile
  kVarMid = 1,      // WQ=4, WK=1: 4 query rows
  kVarDecode = 2,   // WQ=2, WK=2: 2 query rows, two waves per row split the keys
  kVarQuant = 3,    // WQ=4, WK=1: 4 query rows, fp8 / int8 sequences of more than 4 rows
};
constexpr int kVariantTileQ[4] = {8, 4, 2, 4};
constexpr int kVariantWaves[4] = {8, 4, 4, 4};
// Keys per staged tile: 256 for prefill (half the stage barriers per MFMA of
// 128-key tiles, 1.4% faster on a causal 8K prefill although its eight query
// rows, 128 KB at D = 128, then no longer fit in LDS beside a stage), 128 for
// the two-per-CU variants, whose LDS holds two stages at most.
constexpr int kVariantTileK[4] = {256, 128, 128, 128};

// Buffer resource word 3 for raw (untyped) buffer access on gfx9-family GPUs.
// With a zero stride, a lane whose byte offset is >= the record count reads 0
// and has its store dropped by the hardware: masked stores need no branch.
constexpr int kRsrcWord3 = 0x00020000;

// ---------------------------------------------------------------------------
// Kernel arguments
// ---------------------------------------------------------------------------
struct ScoreArgs {
  const uint8_t* q;
  const uint8_t* k;
  const void* w;
  const float* q_scale;
  const float* k_scale;
  const int32_t* block_table;
  const BatchRec* batches;
  const WorkItem* items;
  float* ws;
  int64_t k_block_stride;  // elements between paged blocks
  int64_t num_blocks;      // paged blocks; ids outside [0, num_blocks) are clamped into it
  int32_t n1;              // query heads (== G since N2 == 1)
  int32_t layout_k;
  int32_t dtype_w;
  int32_t block_size;
  int32_t block_shift;     // log2(block_size) when it is a power of two, else -1
  int32_t max_blocks;
  int32_t sparse_mode;
  int32_t cmp_ratio;       // 1 for uncompressed keys
  int32_t key_block;       // keys per stored score (block_len; 1: one score per key)
  int32_t key_block_shift; // log2(key_block)
};

struct TopkArgs {
  const float* ws;
  const RowRec* rows;
  int32_t* out_idx;
  float* out_val;          // may be null
  float* cand_val;         // candidate lists of split rows (workspace), or null
  int32_t* cand_idx;
  int64_t cand_val_off;    // workspace float offset of cand_val
  int32_t k;
  int32_t init_num;        // leading blocks of every row that are always returned
  int32_t local_num;       // trailing visible blocks of every row that are always returned
  int32_t row_class[2 * kTopkClasses + 1];   // pass / class boundaries in records (host copy)
};

// Host launchers (defined next to their kernels).
hipError_t launch_score(const li_problem& p, int variant, int num_items, const ScoreArgs& a,
                        hipStream_t s);
hipError_t launch_topk(const li_problem& p, const TopkArgs& a, hipStream_t s);

// Records the message li_last_error() returns on this thread and returns st.
li_status set_error(li_status st, const char* fmt, ...);

// Visible keys of query row i (i < s_q) of a sequence with lengths (s_q, s_k):
// mode 0 every key; mode 3 the right-down causal rule j <= i + S_k - S_q. With
// compressed keys (ratio r, residual res) the sequence has L = s_k*r + res
// original tokens and compressed key j (tokens j*r .. j*r + r - 1) is visible
// once its last token is: the first floor((i + 1 + L - s_q) / r) keys.
__host__ __device__ inline int32_t visible_keys(int32_t i, int32_t s_q, int32_t s_k, int32_t mode,
                                                int32_t cmp_ratio = 1, int32_t cmp_res = 0) {
  if (mode == 0) return s_k;
  const int64_t num = (int64_t)i + 1 + (int64_t)s_k * cmp_ratio + cmp_res - (int64_t)s_q;
  if (num < cmp_ratio) return 0;
  const int64_t v = num / cmp_ratio;
  return v > s_k ? s_k : (int32_t)v;
}

}  // namespace li
