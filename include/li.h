/*
 * li.h -- C ABI of the MI355X (gfx950) LightningIndexer forward pass.
 *
 * For every query token the library scores every visible key,
 *
 *     s_j = sum_g W[g] * ReLU(Q_index[g] . K_index[j])                (fp16 / bf16)
 *     s_j = sum_g W[g] * ReLU(Sq[g] * Sk[j] * (Qc[g] . Kc[j]))        (fp8-e4m3fn / int8)
 *
 * and returns the top-k keys of each row: int32 sparse_indices and optional
 * float32 sparse_values. The formula and the operand shapes are those of the
 * MindSpore "mindspore.ops.lightning_indexer" page (formula block, parameter
 * list); the quantised form is the VllmQuantLightningIndexer README's
 * (function description formula, parameter table); the two-call protocol
 * (a metadata call that balances the work, then the main call) follows the
 * CANN "LightningIndexerV2" guide (interface split, prototype section).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every call returns li_status. LI_OK is 0, errors are negative. On error
 *   nothing has been enqueued and li_last_error() describes the cause.
 * - The caller owns every buffer. The library never allocates or frees device
 *   memory and keeps no device state between calls.
 * - "host" pointers are read on the CPU during the call; "device" pointers are
 *   only handed to kernels. All device work is enqueued on the caller's HIP
 *   stream and the call returns before it completes.
 * - Inputs must be contiguous in the shapes given below (row-major, last axis
 *   fastest), except the paged key cache whose block axis may be strided.
 * - No C++ exception crosses this interface.
 *
 * Readings of points the pages leave open (also listed in the design notes):
 * keys are ranked by score, ties going to the lower key index; each output row
 * is sorted by descending score; indices are 0-based key positions within the
 * sequence (logical position for the paged layout), plus the batch's
 * output_idx_offset when one is given; unused slots hold -1 in sparse_indices
 * and -inf in sparse_values; query rows past a sequence's actual length are all
 * unused slots; dequant scales must be >= 0 (they are absmax / qmax by
 * construction); NaN inputs give undefined rankings; with compressed keys
 * (cmp_ratio r > 1), compressed key j stands for original tokens
 * j*r .. j*r + r - 1 of a sequence of S_k*r + cmp_residual_k original tokens
 * and is visible under the right-down rule once its last token is; with key
 * blocks (block_len L > 1) block c holds keys c*L .. c*L + L - 1, scores the
 * maximum over its visible keys and is visible when one of its keys is; the
 * blocks always kept (init_num first, local_num last visible) fill the first
 * output slots in ascending block order, the rest follow by score.
 */
#ifndef LI_H_
#define LI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LI_API_VERSION 4

typedef enum li_status {
  LI_OK = 0,
  LI_ERR_INVALID_ARGUMENT = -1,   /* a value or pointer breaks a documented rule   */
  LI_ERR_UNSUPPORTED = -2,        /* legal on the pages, not built here (e.g. N2>1) */
  LI_ERR_EMPTY_TENSOR = -3,       /* an input or output has a zero-sized axis       */
  LI_ERR_WORKSPACE_TOO_SMALL = -4,
  LI_ERR_METADATA_MISMATCH = -5,  /* metadata was built for another problem         */
  LI_ERR_HIP = -6,                /* the HIP runtime reported an error              */
  LI_ERR_BUFFER_TOO_SMALL = -7    /* host metadata buffer too small                 */
} li_status;

typedef enum li_layout {
  LI_LAYOUT_BSND = 0,     /* (B, S, N, D)                                          */
  LI_LAYOUT_TND = 1,      /* (T, N, D), sequences packed, delimited by cu_seqlens  */
  LI_LAYOUT_PA_BSND = 2   /* keys only: (block_count, block_size, N2, D) + block_table */
} li_layout;

typedef enum li_dtype {
  LI_DTYPE_F16 = 0,
  LI_DTYPE_BF16 = 1,
  LI_DTYPE_F32 = 2,
  LI_DTYPE_E4M3FN = 3,    /* OCP FP8 E4M3FN: bias 7, max 448, no inf */
  LI_DTYPE_I8 = 4
} li_dtype;

/*
 * Problem description (plain values, no pointers).
 *
 *  layout_q      LI_LAYOUT_BSND: q (B,S1,N1,D), w (B,S1,N1), outputs (B,S1,N2,k)
 *                LI_LAYOUT_TND : q (T1,N1,D),   w (T1,N1),   outputs (T1,N2,k)
 *  layout_k      BSND: k (B,S2,N2,D); TND: k (T2,N2,D); PA_BSND: k (num_blocks,
 *                block_size, N2, D). Non-paged key layouts must equal layout_q
 *                (MindSpore page, note on layout_key; V2 guide, layout table).
 *  dtype_qk      q and k share it (V2 guide constraint list): F16, BF16, E4M3FN, I8.
 *  dtype_w       F16, BF16 or F32, independent of dtype_qk (the pages disagree;
 *                the quantised README pairs fp8 codes with fp32 weights).
 *  dtype_scale   F32; used only for E4M3FN / I8. q_scale is (B,S1,N1) or (T1,N1);
 *                k_scale has k's shape without D: (B,S2,N2), (T2,N2) or
 *                (num_blocks, block_size, N2) -- per token and head.
 *  batch         B >= 1.
 *  s1, s2        BSND sequence dims of q and k; ignored for TND (0 allowed).
 *  t1, t2        TND row counts of q and k; ignored otherwise.
 *  n1, n2, d     1 <= n1 <= 64, n2 == 1, d in {64, 128} (the pages allow only
 *                d = 128 for the product; the TileLang test shape uses 64).
 *  block_size    PA only: multiple of 16, 16..1024 (V2 guide; quant README).
 *  num_blocks    PA only: blocks in the key cache.
 *  max_blocks_per_seq  PA only: second dim of block_table; must cover the
 *                longest sequence (quant README constraint list).
 *  k_block_stride PA only: elements between consecutive blocks of k (0 means
 *                block_size*n2*d); models the quant README's "stride" attribute.
 *  sparse_count  k, 1..8192 (MindSpore page: up to 2048; the V2 guide's
 *                constraint list: up to 8192).
 *  sparse_mode   0 (every key of the sequence) or 3 (right-down causal: key j is
 *                visible to query row i iff j <= i + S_k - S_q, with the actual
 *                per-sequence lengths).
 *  pre_tokens, next_tokens  reserved by the pages; only INT64_MAX is accepted.
 *  return_value  0: sparse_values may be NULL; 1: sparse_values (float32, same
 *                shape as sparse_indices) is written.
 *  cmp_ratio     key compression ratio r of the V2 guide (cmp_ratio attribute):
 *                0 or 1 = keys are not compressed; 2..128 = k holds compressed
 *                keys (S_k of them per sequence, lengths given in compressed
 *                keys) and, in sparse_mode 3, cmp_residual_k gives each
 *                sequence's leftover original tokens (row i then sees the first
 *                clamp(floor((i + 1 + S_k*r + res - S_q) / r), 0, S_k) keys).
 *  block_len     key-block granularity of the selection (the ops-transformer
 *                issue, LightningIndexer family: block_len 1/2/4/8/16): 0 or 1 =
 *                single keys; 2, 4, 8, 16 = the top-k runs over blocks of that
 *                many consecutive (compressed) keys, block score = the largest
 *                score among the block's visible keys, output indices = block
 *                indices (k then counts blocks).
 *  init_num      >= 0: the first init_num visible blocks (sink tokens in the
 *                issue's words) are always returned.
 *  local_num     >= 0: the last local_num visible blocks of each row (the
 *                issue's diagonal local window: under sparse_mode 3 they end at
 *                the row's diagonal) are always returned.
 *                init_num + local_num <= sparse_count. The blocks always kept
 *                take the first output slots, ascending; the other slots hold
 *                the best remaining blocks by (score desc, index asc).
 */
typedef struct li_problem {
  uint32_t api_version;   /* LI_API_VERSION */
  int32_t layout_q;
  int32_t layout_k;
  int32_t dtype_qk;
  int32_t dtype_w;
  int32_t dtype_scale;
  int32_t batch;
  int32_t s1;
  int32_t s2;
  int32_t n1;
  int32_t n2;
  int32_t d;
  int64_t t1;
  int64_t t2;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int64_t num_blocks;
  int64_t k_block_stride;
  int32_t sparse_count;
  int32_t sparse_mode;
  int64_t pre_tokens;
  int64_t next_tokens;
  int32_t return_value;
  int32_t cmp_ratio;
  int32_t block_len;
  int32_t init_num;
  int32_t local_num;
  int32_t reserved[3];    /* must be zero */
} li_problem;

/*
 * Sequence lengths, HOST pointers, read only by li_metadata (the V2 guide's
 * SeqLengths group and the MindSpore actual_seq_lengths_* arguments).
 *
 *  cu_seqlens_q  (B+1) int32: TND query prefix sums, first 0, non-decreasing,
 *                last == t1. Required for TND queries, rejected for BSND.
 *  cu_seqlens_k  (B+1) int32: same for TND keys. Required for TND keys,
 *                rejected for BSND and PA_BSND.
 *  seqused_q     (B) int32, optional: actual query length of each batch, <= s1
 *                (BSND) or <= the cu_seqlens_q length (TND); rows past it are
 *                unused (all -1 / -inf; under TND this is the V2 guide's "TND
 *                Padding" of its constraint list), and the causal rule takes
 *                it as S_q. NULL means the full length.
 *  seqused_k     (B) int32: actual key lengths. Optional for BSND (<= s2) and
 *                TND (<= the cu_seqlens_k length), NULL meaning the full length;
 *                required for PA_BSND (covered by max_blocks_per_seq blocks).
 *  cmp_residual_k (B) int32: original tokens past the last whole compressed key
 *                of each sequence, 0 <= res < cmp_ratio (V2 guide, cmp_residual_k).
 *                Required when cmp_ratio > 1 and sparse_mode == 3, else NULL.
 *  output_idx_offset (B) int32, optional: a value >= 0 added to every returned
 *                index of the sequence's rows (-1 slots unchanged); every
 *                key index + offset must fit in int32 (V2 guide, output_idx_offset).
 */
typedef struct li_lengths {
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  const int32_t* seqused_q;
  const int32_t* seqused_k;
  const int32_t* cmp_residual_k;
  const int32_t* output_idx_offset;
} li_lengths;

/*
 * Operands, DEVICE pointers (shapes and dtypes as in li_problem).
 *  q, k, w       required.
 *  q_scale, k_scale  float32 dequant scales, required for E4M3FN / I8, else NULL.
 *  block_table   (B, max_blocks_per_seq) int32 physical block ids, required for
 *                PA_BSND; entries past a sequence's last block are never read.
 *                Ids outside [0, num_blocks) are clamped into that range (no
 *                fault; the scores of the keys they cover are then unspecified).
 */
typedef struct li_inputs {
  const void* q;
  const void* k;
  const void* w;
  const float* q_scale;
  const float* k_scale;
  const int32_t* block_table;
} li_inputs;

/*
 * li_metadata -- host-only work partitioner (the V2 guide's metadata call).
 *
 * Validates the problem and the lengths (the guide's checker rules) and writes
 * an opaque task table into meta_host: per-sequence records and work items of
 * (sequence, query-row tile, key range), ordered heaviest first so that the
 * CUs stay busy under causal and varlen imbalance. The table also carries a
 * hash of the problem; the compute calls reject a table built for another one.
 *
 *  num_cus       compute units to balance for (256 on MI355X; <= 0 means 256).
 *  meta_host     host buffer of meta_capacity bytes, or NULL to query the size.
 *  meta_bytes    out: bytes needed / written.
 *
 * The caller copies the meta_bytes bytes to device memory (16-byte aligned)
 * for the compute calls and keeps the host copy: both are passed.
 * Returns LI_ERR_BUFFER_TOO_SMALL (with *meta_bytes set) if meta_capacity is short.
 */
li_status li_metadata(const li_problem* p, const li_lengths* lengths, int32_t num_cus,
                      void* meta_host, size_t meta_capacity, size_t* meta_bytes);

/*
 * li_workspace_size -- host-only: bytes of device workspace li_score/li_indexer
 * need: the head-reduced float32 scores of every visible (row, key) pair and,
 * when the task table splits long rows (few rows, k <= 2048), the candidate
 * lists that li_topk passes between its two passes. This is the first half of
 * the two-stage pattern the V2 guide describes for the aclnn interface
 * ("与其他调用方式的关系": a GetWorkspaceSize call, then the launch with the
 * caller's workspace).
 *  meta_host     the table li_metadata wrote for this same problem.
 *  bytes         out: workspace bytes (at least 4).
 * Errors: LI_ERR_METADATA_MISMATCH if the table was built for another problem
 * (any field hashed into it, sparse_count, init_num and local_num included).
 */
li_status li_workspace_size(const li_problem* p, const void* meta_host, size_t* bytes);

/*
 * li_score -- enqueue the score kernel: s_j for every visible (row, key) pair,
 * written as float32 into the workspace (layout private to the library). The
 * score is the MindSpore page's formula block (the sum over heads of
 * W * ReLU(q . k)), the quantised README's function-description formula for
 * E4M3FN / I8, with the V2 guide's visibility rules (sparse_mode, actual
 * lengths, cmp_ratio).
 *  in            device operands (see li_inputs).
 *  meta_host / meta_dev  the same table, on the host and on the device
 *                (16-byte aligned); only meta_host is read by the call.
 *  ws, ws_bytes  device workspace of at least li_workspace_size() bytes,
 *                16-byte aligned; q and k must be 16-byte aligned too.
 *  stream        hipStream_t (NULL = default stream).
 * Errors (nothing enqueued): LI_ERR_INVALID_ARGUMENT for a missing operand or
 * a misaligned pointer, LI_ERR_METADATA_MISMATCH, LI_ERR_WORKSPACE_TOO_SMALL,
 * LI_ERR_HIP if the launch fails.
 */
li_status li_score(const li_problem* p, const li_inputs* in, const void* meta_host,
                   const void* meta_dev, void* ws, size_t ws_bytes, void* stream);

/*
 * li_topk -- enqueue the per-row top-k over a workspace filled by li_score:
 * the k largest scores of each row, sorted by descending score, equal scores
 * by ascending key index (the V2 guide asks for a deterministic result,
 * "确定性计算"; the TileLang guide's golden takes the largest k, sorted), the
 * unused slots holding -1 / -inf (V2 guide, constraint list).
 *  meta_host / meta_dev  as for li_score.
 *  ws, ws_bytes    the workspace li_score filled; the scores are only read, the
 *                  candidate-list part (split rows) is written.
 *  sparse_indices  device int32, (B,S1,N2,k) or (T1,N2,k).
 *  sparse_values   device float32 of the same shape; required iff return_value.
 * Errors (nothing enqueued): LI_ERR_INVALID_ARGUMENT (missing output, values
 * requested without a buffer, misaligned workspace), LI_ERR_METADATA_MISMATCH,
 * LI_ERR_WORKSPACE_TOO_SMALL, LI_ERR_HIP.
 */
li_status li_topk(const li_problem* p, const void* meta_host, const void* meta_dev,
                  void* ws, size_t ws_bytes, int32_t* sparse_indices,
                  float* sparse_values, void* stream);

/*
 * li_indexer -- li_score followed by li_topk on the same stream: the whole
 * operator of the MindSpore page's signature (query, key, weights, lengths,
 * block table, sparse_count, sparse_mode, return_value) with the workspace and
 * task table of the V2 guide's two-call protocol. Both halves are validated
 * before either is enqueued; arguments and errors as for li_score and li_topk.
 */
li_status li_indexer(const li_problem* p, const li_inputs* in, const void* meta_host,
                     const void* meta_dev, void* ws, size_t ws_bytes,
                     int32_t* sparse_indices, float* sparse_values, void* stream);

/*
 * li_indexer_noalloc -- li_indexer without a caller workspace, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. The call allocates nothing;
 * its workspace is a device array inside the library of li_noalloc_capacity()
 * bytes (256 MiB: an 8K x 8K causal prefill fits), held by every GPU the
 * library runs on until the process ends.
 *  Arguments as for li_indexer, without ws / ws_bytes.
 * Errors: as for li_indexer; LI_ERR_WORKSPACE_TOO_SMALL (nothing enqueued)
 * when li_workspace_size() of the problem exceeds the capacity; LI_ERR_HIP if
 * the array's device address cannot be obtained.
 * All calls on one GPU share that GPU's array: calls that may overlap on one
 * GPU (different streams or threads without ordering) race and give undefined
 * results; calls ordered on one stream are safe. Nothing in the array needs to
 * be cleared between calls.
 */
li_status li_indexer_noalloc(const li_problem* p, const li_inputs* in, const void* meta_host,
                             const void* meta_dev, int32_t* sparse_indices,
                             float* sparse_values, void* stream);

/* Bytes of the device array li_indexer_noalloc uses as its workspace. */
size_t li_noalloc_capacity(void);

/* Message for the last non-OK status returned on the calling thread. */
const char* li_last_error(void);

/* LI_API_VERSION of the built library. */
int32_t li_api_version(void);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* LI_H_ */
