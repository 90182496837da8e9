// Score kernel: s_j = sum_g W[g] * ReLU(Q[g] . K[j]) for every visible (row, key)
// pair, head-reduced in registers so that one float per pair leaves the CU.
//
// The formula is the indexer formula of the MindSpore lightning_indexer page
// (formula block) and, for fp8 / int8 codes with per-token-head dequant scales,
// of the VllmQuantLightningIndexer README (function description): there the
// scales enter as ReLU(Sq[g]*Sk[j]*(Qc[g].Kc[j])). Scales are non-negative, so
// this equals Sk[j] * sum_g (W[g]*Sq[g]) * ReLU(Qc[g].Kc[j]), which is what the
// kernel evaluates: W*Sq is folded per head at load, Sk multiplies the reduced
// score once per key.
//
// Work decomposition (one workgroup per work item of the task table):
//   * the workgroup owns WQ query rows of one sequence and a key range [k0,k1);
//   * WQ rows x WK key slices of waves, two waves per SIMD so that one can issue
//     while the other waits: 8 waves in one workgroup per CU for prefill tiles,
//     4 waves in each of two workgroups per CU for short sequences (one
//     workgroup's start then overlaps the other's key loop), and for fp8 / int8
//     prefill 4 waves in each of three workgroups per CU (below); a wave holds its
//     row's query heads in VGPRs as MFMA A-operands for the whole key loop
//     (16-bit D = 128 rows arrive through LDS as coalesced blocks, others by
//     direct loads);
//   * keys are staged KT at a time in two LDS buffers by direct global -> LDS
//     loads (no staging registers), gathered through the block table for the
//     paged layout;
//   * per 32-key slice a wave runs NT x (D / k-step) MFMA 32x32 ops with heads on
//     the M axis and keys on the N axis, with B fragments read one slice ahead;
//     each lane then holds 16 heads of one key per tile, applies ReLU and the
//     per-head weight (interleaved with the next slice's MFMAs: two accumulator
//     sets, PP), and one cross-lane swap-add over the two half-waves completes
//     the reduction. fp8 / int8 MFMAs cover a slice in a quarter of the bf16
//     count, so there the epilogue's two VALU operations per (head, key) bound
//     the kernel; that variant keeps one accumulator set (PP = false: a slice's
//     epilogue runs before the next slice's MFMAs), which brings it to 168
//     VGPRs and three waves per SIMD, and the waves hide each other's wait for
//     MFMA results (5.53 -> 5.27 ms on a 16-sequence fp8 prefill, identical
//     outputs; on 4-row fp8 decode it was 6% slower, so kVarMid keeps PP);
//   * with key blocks (block_len > 1) the maximum over each block's visible keys
//     is taken across lanes before the store, so one float per block leaves.
#include "li_internal.h"

#include <utility>

namespace li {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// One MFMA family per storage dtype. All produce a 32x32 tile in which lane l
// holds column (l % 32) and, for accumulator element e, row
// 8*(e/4) + 4*(l/32) + e%4. Operand fragments are kLaneBytes of one A row /
// B column per lane; lanes 0-31 and 32-63 hold the two halves of a k-step.
template <int DT> struct Mma;

template <> struct Mma<LI_DTYPE_BF16> {
  static constexpr int kElemBytes = 2;
  static constexpr int kLaneBytes = 16;
  using Frag = i32x4_t;
  using Acc = f32x16_t;
  __device__ static Acc zero() { return Acc{}; }
  __device__ static Acc mma(Frag a, Frag b, Acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  // ReLU on the float bits: a negative float is a negative int32, so an integer
  // max with 0 gives +0 for it and leaves non-negative values unchanged.
  __device__ static float relu(const Acc& c, int e) {
    return __int_as_float(max(__float_as_int(c[e]), 0));
  }
};

template <> struct Mma<LI_DTYPE_F16> {
  static constexpr int kElemBytes = 2;
  static constexpr int kLaneBytes = 16;
  using Frag = i32x4_t;
  using Acc = f32x16_t;
  __device__ static Acc zero() { return Acc{}; }
  __device__ static Acc mma(Frag a, Frag b, Acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  __device__ static float relu(const Acc& c, int e) {
    return __int_as_float(max(__float_as_int(c[e]), 0));
  }
};

template <> struct Mma<LI_DTYPE_E4M3FN> {
  static constexpr int kElemBytes = 1;
  static constexpr int kLaneBytes = 32;
  using Frag = i32x8_t;
  using Acc = f32x16_t;
  __device__ static Acc zero() { return Acc{}; }
  // Operand formats 0/0 select e4m3 for A and B; zero scale operands select
  // the unscaled form of the instruction.
  __device__ static Acc mma(Frag a, Frag b, Acc c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
  __device__ static float relu(const Acc& c, int e) {
    return __int_as_float(max(__float_as_int(c[e]), 0));
  }
};

template <> struct Mma<LI_DTYPE_I8> {
  static constexpr int kElemBytes = 1;
  static constexpr int kLaneBytes = 16;
  using Frag = i32x4_t;
  using Acc = i32x16_t;
  __device__ static Acc zero() { return Acc{}; }
  __device__ static Acc mma(Frag a, Frag b, Acc c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
  __device__ static float relu(const Acc& c, int e) { return (float)max(c[e], 0); }
};

template <typename F> __device__ inline F load_frag(const uint8_t* p);
template <> __device__ inline i32x4_t load_frag<i32x4_t>(const uint8_t* p) {
  return *reinterpret_cast<const i32x4_t*>(p);
}
template <> __device__ inline i32x8_t load_frag<i32x8_t>(const uint8_t* p) {
  return *reinterpret_cast<const i32x8_t*>(p);
}

__device__ inline float load_weight(const void* w, int dtype, int64_t i) {
  if (dtype == LI_DTYPE_F32) return static_cast<const float*>(w)[i];
  const uint16_t bits = static_cast<const uint16_t*>(w)[i];
  if (dtype == LI_DTYPE_BF16) return __uint_as_float(uint32_t(bits) << 16);
  return (float)__builtin_bit_cast(_Float16, bits);
}

// The key-row swizzle of the score kernel's LDS tiles (see there), as a
// compile-time function of the row for rows of ROW bytes.
template <int ROW> constexpr int swz_of(int r) {
  constexpr int U = ROW / 16;
  constexpr int RPW = ROW >= 128 ? 1 : 128 / ROW;   // key rows per 128-byte bank window
  const int x = r / RPW;
  return (x ^ (x >> __builtin_ctz(U))) & (U - 1);
}

// Byte offset past any record count: the store is dropped (kRsrcWord3).
constexpr int kDropOffset = (int)0x80000000u;

template <int N, typename F, int... I>
__device__ inline void unroll_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F> __device__ inline void unroll(F&& f) {
  unroll_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// Direct global -> LDS load of 16 bytes per lane: lane i of the wave writes
// LDS bytes [lds + 16 i, lds + 16 i + 16). The LDS base is wave-uniform (M0).
// Issued from asm so that the compiler's own wait-count bookkeeping does not
// treat the in-flight staging buffer as aliasing the one being read; the
// completion wait is explicit (stage_barrier). No VGPR is written.
__device__ inline void lds_dma16(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds), "v"(gptr)
               : "memory", "m0");
}

// The same from a wave-uniform base address plus a 32-bit per-lane byte offset
// (the scalar-base form: no 64-bit address arithmetic per lane).
__device__ inline void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// v from the lane that a DPP permutation inside 16-lane rows selects.
template <int CTRL> __device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Max over aligned groups of `len` consecutive lanes (len in 1..16, a power of
// two): xor-1 and xor-2 quad permutations, then the half-row and row mirrors,
// which pair the two halves of each 8- and 16-lane group.
__device__ inline float group_max(float v, int len) {
  if (len >= 2) v = fmaxf(v, dpp<0xB1>(v));     // quad_perm [1,0,3,2]
  if (len >= 4) v = fmaxf(v, dpp<0x4E>(v));     // quad_perm [2,3,0,1]
  if (len >= 8) v = fmaxf(v, dpp<0x141>(v));    // row_half_mirror
  if (len >= 16) v = fmaxf(v, dpp<0x140>(v));   // row_mirror
  return v;
}

// Wait until at most N vector-memory operations of this wave are outstanding
// and all its LDS operations are done, then barrier the workgroup.
template <int N> __device__ inline void stage_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

// BL: store one score per block of block_len keys (the block maximum) instead
// of one per key.
template <int DT, int D, int NT, int WQ, int WK, int KT, bool BL, bool PP = true,
          int MINB = (WQ * WK == 4 ? 2 : 1)>
__global__ __launch_bounds__(WQ * WK * 64, MINB) void score_kernel(ScoreArgs a) {
  using M = Mma<DT>;
  using Frag = typename M::Frag;
  using Acc = typename M::Acc;
  constexpr int ES = M::kElemBytes;
  constexpr int LB = M::kLaneBytes;
  constexpr int ROW = D * ES;              // bytes of one key row
  constexpr int KSTEPS = ROW / (2 * LB);   // MFMA k-steps over the head dim
  constexpr int NW = WQ * WK;              // waves
  constexpr int NTHR = NW * 64;
  constexpr int STAGE = KT * ROW;          // bytes of one staged key tile
  constexpr int DMA = STAGE / 1024;        // 1 KB wave loads per stage
  constexpr int DPW = DMA / NW;            // ... per wave
  constexpr int U = ROW / 16;              // 16-byte swizzle units per key row
  constexpr int NU = LB / 16;              // units per lane fragment (1 or 2)
  constexpr bool QUANT = (DT == LI_DTYPE_E4M3FN) || (DT == LI_DTYPE_I8);
  constexpr int SPS = KT / 32 / WK;        // 32-key slices per staged tile per wave
  constexpr int EPM = 16 / KSTEPS;         // previous-slice accumulators per MFMA
  static_assert(KT % (32 * WK) == 0 && SPS % 2 == 0, "a stage holds an even number of slices");
  static_assert(KSTEPS >= 1 && ROW % (2 * LB) == 0, "head dim must fill whole k-steps");
  static_assert(STAGE % (1024 * NW) == 0, "every wave stages the same number of 1 KB blocks");
  static_assert((ROW & (ROW - 1)) == 0 && (U & (U - 1)) == 0 && NU * 16 == LB, "power-of-two rows");
  static_assert(!QUANT || KT + 32 <= NTHR, "one thread per staged key scale and its copy");
  // Query rows of 256-byte heads (16-bit D = 128) are staged through LDS when
  // they fit beside one key stage (160 KB for one workgroup per CU, 80 KB for
  // two): QROW bytes per row (N1 <= 64). Loaded straight into A-operand
  // registers, each 1 KB load of a row touches 32 cache lines (32 bytes of 32
  // heads); staged, it is one coalesced 1 KB block. (Shorter heads gained
  // nothing measurable and keep the direct loads.)
  constexpr int QROW = 64 * ROW;
  constexpr int LDS_CAP = NW == 8 ? 160 * 1024 : 80 * 1024;
  constexpr int QEXTRA = QUANT ? 2 * KT * 4 : 0;
  constexpr bool QLDS = ROW >= 256 && STAGE + WQ * QROW + QEXTRA <= LDS_CAP;
  // The query rows sit after both key stages if they fit there, else over the
  // second stage (which is then loaded once they have been read).
  constexpr bool QOVER = 2 * STAGE + WQ * QROW + QEXTRA > LDS_CAP;
  // Rows too large to sit beside a stage may still fit over both stage buffers:
  // they are then staged and read before the first key stage is loaded.
  constexpr bool QALL = !QLDS && !QUANT && ROW >= 256 && WQ * QROW <= 2 * STAGE;
  constexpr bool QSTAGED = QLDS || QALL;
  constexpr int QOFF = QALL ? 0 : (QOVER ? STAGE : 2 * STAGE);
  constexpr int KBUF = QLDS ? (QOFF + WQ * QROW > 2 * STAGE ? QOFF + WQ * QROW : 2 * STAGE)
                            : 2 * STAGE;

  // Two staged key tiles. Key row r of a tile occupies bytes [r*ROW, (r+1)*ROW);
  // its 16-byte unit u is stored at unit position u ^ swz(r). A fragment read
  // is one or two 16-byte LDS reads per lane, each taking the same unit of 32
  // consecutive rows; with x = r / RPW, swz = (x ^ (x >> log2 U)) mod U puts
  // any 8 (and any 16) consecutive rows of such a read on distinct banks.
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf[KBUF];
  // Key dequant scales in a ring of three stages, stage st at
  // [(st % 3) * KT, +KT), and after them a copy of ring slot 0's first 32: the
  // scales of two consecutive 32-key slices then always lie side by side,
  // also across the end of the ring. Three slots, not two: stage st + 3 is
  // stashed before the barrier ending stage st + 2, and a wave can be one
  // barrier behind the others, so stage st's scales stay readable through
  // stage st + 1 (pairs of slices read them after the barrier ending stage st).
  __shared__ float ksc[QUANT ? 3 * KT + 32 : 1];
  auto swz = [](int r) { return swz_of<ROW>(r); };

  // The LB-byte fragment at LDS byte base ^ (2*LB*s) (and ^16 for its second
  // 16-byte half).
  auto read_frag = [&](int base, int s) {
    const int a = base ^ (2 * LB * s);
    if constexpr (NU == 1) {
      return *reinterpret_cast<const Frag*>(&kbuf[a]);
    } else {
      const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(&kbuf[a]);
      const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(&kbuf[a ^ 16]);
      return Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };

  const WorkItem it = a.items[blockIdx.x];
  const BatchRec br = a.batches[it.b];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wq = wave % WQ;
  const int wk = wave / WQ;
  const int half = lane >> 5;
  const int col = lane & 31;

  const int row = it.q0 + wq;
  const bool row_ok = row < br.s_q;
  const int nv = row_ok ? visible_keys(row, br.s_q, br.s_k, a.sparse_mode, a.cmp_ratio, br.cmp_res)
                        : 0;
  const int lim = nv < it.k1 ? nv : it.k1;   // this row stores keys [k0, lim)
  const int64_t qrow = (int64_t)br.row_base + (row_ok ? row : 0);
  float* out_row = a.ws + br.ws_off + (int64_t)(row_ok ? row : 0) * br.ld;
  // Stored floats of the row: keys [0, lim), or the blocks holding them. Items
  // start at multiples of KT, so no block straddles two items.
  const int nstore = BL ? (lim + a.key_block - 1) >> a.key_block_shift : lim;
  const auto out_rsrc = __builtin_amdgcn_make_buffer_rsrc(out_row, (short)0,
                                                          nstore > 0 ? nstore * 4 : 0, kRsrcWord3);

  // Key staging. Stage st covers keys [k0 + st*KT, k0 + (st+1)*KT); keys past
  // k1 are clamped to the item's last key (computed, never stored), so every
  // load is unconditional. For the paged cache the block ids of a stage are
  // loaded one stage before its keys, with scalar loads: a 1 KB DMA block holds
  // 1024/ROW <= 16 consecutive keys starting at a multiple of 1024/ROW, and cache
  // blocks are multiples of 16 keys, so all its keys (clamped ones included)
  // share one cache block, the one of its first key.
  const bool paged = a.layout_k == LI_LAYOUT_PA_BSND;
  const int jmax = it.k1 - 1;
  const int32_t* btab = a.block_table + (int64_t)it.b * a.max_blocks;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)kbuf;
  // LDS byte (of the wave's d-th 1 KB block) this lane writes, and the key row
  // and byte within the row that belong there.
  auto dma_row = [&](int d, int ln) { return ((d * NW + wave) * 1024 + ln * 16) / ROW; };
  auto dma_byte = [&](int d, int ln) {
    const int r = dma_row(d, ln);
    const int b = (ln * 16) % ROW;   // 1 KB blocks hold whole rows
    return ((b / 16) ^ swz(r)) * 16;
  };
  auto stage_key = [&](int st, int kk) { return min(it.k0 + st * KT + kk, jmax); };
  auto block_index = [&](int j) { return a.block_shift >= 0 ? j >> a.block_shift : j / a.block_size; };
  auto clamp_block = [&](int blk) {
    return blk < 0 ? 0 : (blk >= a.num_blocks ? (int)(a.num_blocks - 1) : blk);
  };
  int pid[DPW];
  int psid = 0;
  const auto* btab_s = (const __attribute__((address_space(4))) int32_t*)btab;
  auto ids = [&](int st) {
    if (!paged) return;
#pragma unroll
    for (int d = 0; d < DPW; ++d)
      pid[d] = btab_s[block_index(stage_key(st, (d * NW + wave) * 1024 / ROW))];
    if (QUANT) psid = btab[block_index(stage_key(st, tid % KT))];
  };
  float pre_sc = 0.f;
  // Within a contiguous stage, the lane's d-th 1 KB DMA block reads from byte
  // (d * NW + wave) * 1024 + (dma_v ^ 16 * swz(R_d)), R_d = (d * NW + wave) *
  // 1024 / ROW its first key row: 1 KB blocks hold whole rows, and the
  // swizzle of a row R_d + l (l < 1024 / ROW, R_d a multiple of it) is
  // swz(R_d) ^ swz(l) for every row size here, so the block's part of the
  // source offset is a uniform XOR of the lane's offset in block 0.
  const uint32_t dma_v = (uint32_t)((lane * 16 / ROW) * ROW +
                                    ((((lane * 16) % ROW) / 16) ^ swz(lane * 16 / ROW)) * 16);
  const auto ks_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.k_scale) + (QUANT ? br.k_base : 0), (short)0, QUANT ? br.s_k * 4 : 0,
      kRsrcWord3);
  auto fetch = [&](int st) {
    const uint32_t lds = lds0 + (st & 1) * STAGE;
    if (!paged && it.k0 + (st + 1) * KT <= it.k1) {   // uniform
      // A whole contiguous stage (no key clamped): each block is a scalar base
      // plus the lane's offset, one XOR per block. The opaque copy keeps the
      // per-block offsets from being hoisted out of the stage loop (DPW more
      // live registers).
      const uint8_t* sb = a.k + ((int64_t)br.k_base + it.k0 + st * KT) * ROW;
      uint32_t v = dma_v;
      asm volatile("" : "+v"(v));
#pragma unroll
      for (int d = 0; d < DPW; ++d) {
        const int blk = d * NW + wave;
        lds_dma16_s(sb + blk * 1024, v ^ (16u * (uint32_t)swz(blk * (1024 / ROW))), lds + blk * 1024);
      }
      if (QUANT)
        pre_sc = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            ks_rsrc, (uint32_t)(tid % KT) * 4u, (it.k0 + st * KT) * 4, 0));
      return;
    }
    if (!paged) {
      // The last stage of an item (keys clamped to its last key). The opaque
      // lane keeps this path's per-block rows and bytes from being hoisted
      // out of the stage loop, where they would hold registers for a path
      // taken once per item.
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int d = 0; d < DPW; ++d) {
        const int64_t off = ((int64_t)br.k_base + stage_key(st, dma_row(d, ln))) * ROW;
        lds_dma16(a.k + off + dma_byte(d, ln), lds + (d * NW + wave) * 1024);
      }
      if (QUANT) pre_sc = a.k_scale[(int64_t)br.k_base + stage_key(st, tid % KT)];
      return;
    }
    // Paged keys: each block's source is its cache block's row. (The
    // one-accumulator-set kernels have no registers to spare for hoisted lane
    // offsets: opaque lane there too.)
    int lp = lane;
    if constexpr (!PP) asm volatile("" : "+v"(lp));
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
      const int j = stage_key(st, dma_row(d, lp));
      const int bo = j - block_index(j) * a.block_size;
      const int64_t off = ((int64_t)clamp_block(pid[d]) * a.k_block_stride + (int64_t)bo * D) * ES;
      lds_dma16(a.k + off + dma_byte(d, lp), lds + (d * NW + wave) * 1024);
    }
    if (QUANT) {
      const int j = stage_key(st, tid % KT);
      pre_sc = a.k_scale[(int64_t)clamp_block(psid) * a.block_size + (j - block_index(j) * a.block_size)];
    }
  };
  auto stash_scales = [&](int st) {
    const int sr = st % 3;   // ring slot (uniform)
    if (QUANT && tid < KT) ksc[sr * KT + tid] = pre_sc;
    // threads KT .. KT+31 hold the scales of keys 0 .. 31 of the stage
    if (QUANT && sr == 0 && tid >= KT && tid < KT + 32) ksc[3 * KT + tid - KT] = pre_sc;
  };

  const int nstages = (it.k1 - it.k0 + KT - 1) / KT;
  ids(0);
  if (!QALL) fetch(0);
  if (!(QLDS && QOVER)) stash_scales(0);
  Frag qf[NT][KSTEPS];
  if constexpr (QSTAGED) {
    // The row's N1 x ROW query bytes go to LDS as coalesced 1 KB blocks (split
    // over the row's WK waves), head h laid out like key row h, and come back
    // as A-operands with the key fragments' conflict-free reads. Bytes past the
    // row's heads (clamped source) land in padded heads, which are masked.
    const int qbytes = a.n1 * ROW;
    const uint8_t* qsrc = a.q + qrow * (int64_t)qbytes;
    const uint32_t qlds = lds0 + QOFF + wq * QROW;
    for (int bk = wk; bk * 1024 < qbytes; bk += WK) {
      const int L = bk * 1024 + lane * 16;
      const int h = L / ROW;
      const int g = h * ROW + (((L % ROW) / 16) ^ swz(h)) * 16;
      lds_dma16(qsrc + (g < qbytes ? g : qbytes - 16), qlds + bk * 1024);
    }
  } else {
    if (nstages > 1) {
      ids(1);
      fetch(1);
    }
    // Query heads of this row as MFMA A-operands (zero for padded heads). Every
    // load is unconditional (clamped index, masked afterwards) so that they are
    // all in flight together with the first key tiles.
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int h = 32 * t + col;
      const bool ok = row_ok && h < a.n1;
      const uint8_t* src = a.q + ((qrow * a.n1 + (ok ? h : 0)) * D) * ES + half * LB;
      const int mask = ok ? -1 : 0;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qf[t][s] = load_frag<Frag>(src + s * 2 * LB) & mask;
    }
  }
  if (QLDS && nstages > 1) {
    ids(1);
    if (!QOVER) fetch(1);
  }
  if (!(QLDS && QOVER) && !QALL && nstages > 2) ids(2);
  // The per-lane weights of the 16 heads each lane accumulates per tile.
  float wr[NT][16];
  {
    int64_t widx[NT][16];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int he = 32 * t + 8 * (e >> 2) + 4 * half + (e & 3);
        widx[t][e] = qrow * a.n1 + (he < a.n1 ? he : a.n1 - 1);
      }
    if (a.dtype_w == LI_DTYPE_F32) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) wr[t][e] = static_cast<const float*>(a.w)[widx[t][e]];
    } else {
      uint16_t raw[NT][16];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) raw[t][e] = static_cast<const uint16_t*>(a.w)[widx[t][e]];
      const bool is_bf16 = a.dtype_w == LI_DTYPE_BF16;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          wr[t][e] = is_bf16 ? __uint_as_float(uint32_t(raw[t][e]) << 16)
                             : (float)__builtin_bit_cast(_Float16, raw[t][e]);
    }
    if (QUANT) {
      float qs[NT][16];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) qs[t][e] = a.q_scale[widx[t][e]];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) wr[t][e] *= qs[t][e];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int he = 32 * t + 8 * (e >> 2) + 4 * half + (e & 3);
        wr[t][e] = (row_ok && he < a.n1) ? wr[t][e] : 0.f;
      }
  }
  if constexpr (QSTAGED) {
    // rows staged, weights in registers, and (unless the rows fill both stage
    // buffers) stage 0, and stage 1 if apart from the rows
    stage_barrier<0>();
    if (QOVER) stash_scales(0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int h = 32 * t + col;
      const int mask = (row_ok && h < a.n1) ? -1 : 0;
      const int qb = QOFF + wq * QROW + h * ROW + 16 * ((half * NU) ^ swz(h));
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qf[t][s] = read_frag(qb, s) & mask;
    }
    if constexpr (QALL) {
      stage_barrier<0>();   // query rows read: both stage buffers are free
      fetch(0);
      if (nstages > 1) {
        ids(1);
        fetch(1);
      }
      if (nstages > 2) ids(2);
      if (nstages > 1) stage_barrier<DPW>();   // stage 0 staged (stage 1 may still load)
      else stage_barrier<0>();
    } else if constexpr (QOVER) {
      stage_barrier<0>();   // query rows read (their space takes stage 1), scales published
      if (nstages > 1) fetch(1);
      if (nstages > 2) ids(2);
    }
  } else {
    stage_barrier<0>();   // stage 0 (and 1) staged, query and weights in registers
  }

  // One loop iteration per stage, its SPS slices unrolled. Slice i of stage st
  // covers keys [k0 + st*KT + (wk + i*WK)*32, +32) in buffer st & 1. Before the
  // last slice of a stage every wave has read all it needs of that buffer, so
  // after a barrier (which also publishes the next stage, loaded a stage
  // earlier) the stage after next is loaded into it. Per slice: MFMAs of the
  // slice, each k-step's B fragment reloaded right after use with the next
  // slice's, and the ReLU / weight / in-lane head reduction of the previous
  // slice interleaved between the MFMAs; every second slice, the cross-half
  // swap-add and the store of the two previous slices. The store has no branch,
  // so the vector-memory operations issued after the last key DMA before each
  // barrier are exactly SPS/2 stores (SPS/2 - 1 in the first stage).
  auto slice_key = [&](int st, int i) { return it.k0 + st * KT + (wk + i * WK) * 32; };
  // LDS byte address of this lane's B fragment of k-step s in slice (buf, sub):
  // logical units (2s + half)*NU + e (e < NU) of row r, i.e. the addresses
  // frag_base(buf, sub) ^ (2*LB*s) ^ (16*e), rows being ROW-aligned.
  auto frag_base = [&](int buf, int sub) {
    const int r = sub * 32 + col;
    return buf * STAGE + r * ROW + 16 * ((half * NU) ^ swz(r));
  };
  Frag bf[KSTEPS];
  {
    const int b0 = frag_base(0, wk);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) bf[s] = read_frag(b0, s);
  }
  // Dequant key scale of the next slice, read together with its B fragments.
  float ksn = QUANT ? ksc[wk * 32 + col] : 1.f;
  // FIMM (one key slice per wave, WK == 1, so the slice of every unrolled step
  // is known at compile time): the fragment reads take their slice and k-step
  // from the instruction's immediate offset. The swizzle of row sub*32 + col is
  // swz(col) ^ swz(sub*32), and the logical unit (2s + half)*NU + e is the XOR
  // of its three bit fields, so the physical unit is
  //   ((half*NU) ^ swz(col)) ^ q ^ swz(sub*32),   q = 2*NU*s + e,
  // and XOR with swz(sub*32) permutes the KSTEPS*NU values of q among
  // themselves. fa[m] holds the lane's byte address of value q_m (row col of
  // slice 0, current buffer); a read adds the slice's rows as an immediate. The
  // buffer offset moves with the stages (one add per register per stage, not
  // an address computation per read).
  constexpr int QM = KSTEPS * NU;
  constexpr bool FIMM = WK == 1;
  // FPAIR: two consecutive slices finish together (below) with one scale read
  // and a store offset of one add; their scales are read per pair, not per slice.
  constexpr bool FPAIR = FIMM && !BL;
  auto q_of = [](int m) { return 2 * NU * (m / NU) + m % NU; };
  auto m_of = [](int q) { return (q / (2 * NU)) * NU + q % (2 * NU); };
  uint32_t fa[FIMM ? QM : 1];
  if constexpr (FIMM) {
    const int pl = (half * NU) ^ swz(col);
#pragma unroll
    for (int m = 0; m < QM; ++m) fa[m] = (uint32_t)(col * ROW + 16 * (pl ^ q_of(m)));
  }
  auto step = [&](int st, auto ic, Acc (&acc)[NT], const Acc (&old)[NT], float& ks) {
    constexpr int i = decltype(ic)::value;
    const int buf = st & 1;
    ks = ksn;
    // Next slice: same stage, or the first slice of the next stage (past the
    // last stage this re-reads stale LDS, unused).
    const int nbuf = (i + 1 < SPS) ? buf : (buf ^ 1);
    const int nsub = (i + 1 < SPS) ? wk + (i + 1) * WK : wk;
    const int nbase = frag_base(nbuf, nsub);
    constexpr int NSUB = (i + 1 < SPS) ? i + 1 : 0;   // FIMM (wk == 0)
    if constexpr (FIMM) {
      if constexpr (i + 1 == SPS) {   // the next slice is in the other buffer
        const int dst = buf ? -STAGE : STAGE;
#pragma unroll
        for (int m = 0; m < QM; ++m) fa[m] += (uint32_t)dst;
      }
    }
    // scale of the next slice (stage st, or st + 1 for the last slice)
    if (QUANT && !FPAIR) ksn = ksc[((i + 1 < SPS ? st : st + 1) % 3) * KT + nsub * 32 + col];
    // B fragment of k-step s of the next slice
    auto next_frag = [&](int s) -> Frag {
      if constexpr (FIMM) {
        constexpr int SW = swz_of<ROW>(NSUB * 32);
        i32x4_t h[NU];
#pragma unroll
        for (int e = 0; e < NU; ++e)
          h[e] = *reinterpret_cast<const i32x4_t*>(&kbuf[fa[m_of(q_of(s * NU + e) ^ SW)] +
                                                         NSUB * 32 * ROW]);
        if constexpr (NU == 1) return __builtin_bit_cast(Frag, h[0]);
        else return Frag{h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
      } else {
        return read_frag(nbase, s);
      }
    };
    float p0 = 0.f, p1 = 0.f;
    if constexpr (!PP) {
      // One accumulator set (old aliases acc): the previous slice's epilogue
      // first, in the same order as below, then this slice's MFMAs.
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int u = 0; u < EPM; u += 2) {
            const int e = s * EPM + u;
            // one chain (a second would cost an add per slice; the other
            // waves hide the chain's latency)
            p0 = fmaf(wr[t][e], M::relu(old[t], e), p0);
            p0 = fmaf(wr[t][e + 1], M::relu(old[t], e + 1), p0);
          }
      asm volatile("" : "+v"(p0));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = M::mma(qf[t][s], bf[s], s == 0 ? M::zero() : acc[t]);
        bf[s] = next_frag(s);
      }
      return p0;
    }
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc[t] = M::mma(qf[t][s], bf[s], s == 0 ? M::zero() : acc[t]);
#pragma unroll
        for (int u = 0; u < EPM; u += 2) {
          const int e = s * EPM + u;
          p0 = fmaf(wr[t][e], M::relu(old[t], e), p0);
          p1 = fmaf(wr[t][e + 1], M::relu(old[t], e + 1), p1);
        }
        // Keep this share of the epilogue between its MFMAs: without the pin
        // the IR passes sink the whole ReLU / weight chain behind the last MFMA.
        asm volatile("" : "+v"(p0), "+v"(p1));
        __builtin_amdgcn_sched_barrier(0);
      }
      bf[s] = next_frag(s);
    }
    return p0 + p1;
  };
  // The last slice's epilogue, with the same accumulation order as the one
  // interleaved in step(), so a key's score does not depend on which slice of
  // its item it falls in.
  auto epi = [&](const Acc (&acc)[NT]) {
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int u = 0; u < EPM; u += 2) {
          const int e = s * EPM + u;
          p0 = fmaf(wr[t][e], M::relu(acc[t], e), p0);
          if constexpr (PP) p1 = fmaf(wr[t][e + 1], M::relu(acc[t], e + 1), p1);
          else p0 = fmaf(wr[t][e + 1], M::relu(acc[t], e + 1), p0);
        }
    return PP ? p0 + p1 : p0;
  };
  // Cross-half swap-add (both halves end up with the full sum over heads) and
  // the store of the slice starting at key kb by the lower half-wave; keys at
  // or past the row's limit fall outside the buffer record and are dropped.
  // Stored scores are canonical (x + 0: -0 becomes +0), which the top-k relies on.
  // With blocks, keys past the limit count as -inf in their block's maximum
  // and the first lane of each block stores it.
  auto finish = [&](float part, int kb, float ks, bool valid) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part),
                                                     __float_as_uint(part), false, false);
    float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    tot = QUANT ? fmaf(tot, ks, 0.0f) : tot + 0.0f;   // canonical: never -0
    int off;
    if constexpr (BL) {
      const int j = kb + col;
      tot = group_max(j < lim ? tot : -__builtin_huge_valf(), a.key_block);
      off = (half == 0 && valid && (col & (a.key_block - 1)) == 0) ? (j >> a.key_block_shift) * 4
                                                                    : kDropOffset;
    } else {
      off = (half == 0 && valid) ? (kb + col) * 4 : kDropOffset;
    }
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), out_rsrc, off, 0, 0);
  };
  // Two slices at once: one swap leaves slice A's totals in the lower half-wave
  // and slice B's in the upper one (each added in the same order as above), and
  // one store writes both.
  auto finish2 = [&](float pa, int kba, float ksa, bool valida, float pb, int kbb, float ksb) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pa), __float_as_uint(pb),
                                                     false, false);
    float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    tot = QUANT ? fmaf(tot, half ? ksb : ksa, 0.0f) : tot + 0.0f;   // canonical: never -0
    const int kb = half ? kbb : kba;
    const bool valid = half ? true : valida;
    int off;
    if constexpr (BL) {
      const int j = kb + col;
      tot = group_max(j < lim ? tot : -__builtin_huge_valf(), a.key_block);
      off = (valid && (col & (a.key_block - 1)) == 0) ? (j >> a.key_block_shift) * 4 : kDropOffset;
    } else {
      off = valid ? (kb + col) * 4 : kDropOffset;
    }
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), out_rsrc, off, 0, 0);
  };

  // FPAIR: the same for slices A and B = A + 1 (keys kba and kba + 32), with
  // lane l's key scale read by the caller (ksc bytes of A's first key + 4 l)
  // and lane l's key kba + l; VALID = false drops slice A's half (the first
  // pair of an item, whose slice A does not exist).
  const int lane4 = lane * 4;
  auto finish_pair = [&](float pa, float pb, int kba, float ks, auto valid_tag) {
    constexpr bool VALID = decltype(valid_tag)::value;
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pa), __float_as_uint(pb),
                                                     false, false);
    float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    tot = QUANT ? fmaf(tot, ks, 0.0f) : tot + 0.0f;   // canonical: never -0
    int off = lane4 + kba * 4;
    if constexpr (!VALID) off = half ? off : kDropOffset;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot), out_rsrc, off, 0, 0);
  };
  auto pair_scale = [&](int sbyte) {   // sbyte: ksc byte of slice A's first key
    return QUANT ? *reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(ksc) + sbyte +
                                                   lane * 4)
                 : 1.f;
  };

  // PP: even slices of a stage accumulate in acc0, odd ones in acc1; else all
  // in acc0. The first slice's (dropped) epilogue reads zeros.
  Acc acc0[NT], acc1[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    acc1[t] = M::zero();
    if (!PP) acc0[t] = M::zero();
  }
  float ks0 = 1.f, ks1 = 1.f;
  float hp = 0.f, hks = 1.f;   // an even slice's part, finished with the next one
  int hkb = 0;
  bool hvalid = false;
  for (int st = 0; st < nstages; ++st) {
    unroll<SPS>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (i == SPS - 1) {
        stash_scales(st + 1);   // scales of stage st+1 (ignored past the last stage)
        // one store per two slices since the last key DMA: SPS/2, or one fewer
        // in the first stage (no store from a previous stage)
        if (st == 0) stage_barrier<SPS / 2 - 1>();
        else stage_barrier<SPS / 2>();
        if (st + 2 < nstages) fetch(st + 2);
        if (st + 3 < nstages) ids(st + 3);
      }
      // previous slice: (st, i-1), or the last slice of stage st-1
      const int pkb = i > 0 ? slice_key(st, i - 1) : slice_key(st - 1, SPS - 1);
      if (i % 2 == 0) {
        hp = PP ? step(st, ic, acc0, acc1, ks0) : step(st, ic, acc0, acc0, ks0);
        hkb = pkb;
        hks = ks1;
        hvalid = i > 0 || st > 0;
      } else if constexpr (FPAIR) {
        // slice A = i - 2 of this stage, or (i = 1) the last of the previous
        // one (ring slot (st + 2) % 3; for stage 0 a slot whose lanes are
        // dropped, followed by the copy of stage 0's first 32)
        const float ksp = pair_scale(
            ((i >= 2 ? (st % 3) * KT + (i - 2) * 32 : ((st + 2) % 3) * KT + (SPS - 1) * 32)) * 4);
        const float part = PP ? step(st, ic, acc1, acc0, ks1) : step(st, ic, acc0, acc0, ks1);
        if (i == 1 && st == 0)
          finish_pair(hp, part, hkb, ksp, std::false_type{});
        else
          finish_pair(hp, part, hkb, ksp, std::true_type{});
      } else {
        const float part = PP ? step(st, ic, acc1, acc0, ks1) : step(st, ic, acc0, acc0, ks1);
        finish2(hp, hkb, hks, hvalid, part, pkb, ks0);
      }
    });
  }
  if constexpr (FPAIR) {
    if (QUANT) ks1 = ksc[((nstages - 1) % 3) * KT + (SPS - 1) * 32 + col];
  }
  finish(epi(PP ? acc1 : acc0), slice_key(nstages - 1, SPS - 1), ks1, true);
}

template <int DT, int D, int NT, bool BL>
hipError_t launch_v(int variant, int num_items, const ScoreArgs& a, hipStream_t s) {
  switch (variant) {
    case kVarPrefill:
      hipLaunchKernelGGL((score_kernel<DT, D, NT, 8, 1, kVariantTileK[kVarPrefill], BL>),
                         dim3(num_items), dim3(64 * kVariantWaves[kVarPrefill]), 0, s, a);
      break;
    case kVarMid:
      hipLaunchKernelGGL((score_kernel<DT, D, NT, 4, 1, kVariantTileK[kVarMid], BL>),
                         dim3(num_items), dim3(64 * kVariantWaves[kVarMid]), 0, s, a);
      break;
    case kVarDecode:
      hipLaunchKernelGGL((score_kernel<DT, D, NT, 2, 2, kVariantTileK[kVarDecode], BL>),
                         dim3(num_items), dim3(64 * kVariantWaves[kVarDecode]), 0, s, a);
      break;
    case kVarQuant:
      if constexpr (DT == LI_DTYPE_E4M3FN || DT == LI_DTYPE_I8) {
        hipLaunchKernelGGL((score_kernel<DT, D, NT, 4, 1, kVariantTileK[kVarQuant], BL, false, 3>),
                           dim3(num_items), dim3(64 * kVariantWaves[kVarQuant]), 0, s, a);
        break;
      } else {
        return hipErrorInvalidValue;
      }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT, bool BL>
hipError_t launch_dt(int d, int nt, int variant, int num_items, const ScoreArgs& a, hipStream_t s) {
  if (d == 128) return nt == 1 ? launch_v<DT, 128, 1, BL>(variant, num_items, a, s)
                               : launch_v<DT, 128, 2, BL>(variant, num_items, a, s);
  if (d == 64) return nt == 1 ? launch_v<DT, 64, 1, BL>(variant, num_items, a, s)
                              : launch_v<DT, 64, 2, BL>(variant, num_items, a, s);
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_blk(const ScoreArgs& a, int d, int nt, int variant, int num_items,
                      hipStream_t s) {
  return a.key_block > 1 ? launch_dt<DT, true>(d, nt, variant, num_items, a, s)
                         : launch_dt<DT, false>(d, nt, variant, num_items, a, s);
}

}  // namespace

hipError_t launch_score(const li_problem& p, int variant, int num_items, const ScoreArgs& a,
                        hipStream_t s) {
  if (num_items <= 0) return hipSuccess;
  const int nt = p.n1 > 32 ? 2 : 1;
  switch (p.dtype_qk) {
    case LI_DTYPE_BF16: return launch_blk<LI_DTYPE_BF16>(a, p.d, nt, variant, num_items, s);
    case LI_DTYPE_F16: return launch_blk<LI_DTYPE_F16>(a, p.d, nt, variant, num_items, s);
    case LI_DTYPE_E4M3FN: return launch_blk<LI_DTYPE_E4M3FN>(a, p.d, nt, variant, num_items, s);
    case LI_DTYPE_I8: return launch_blk<LI_DTYPE_I8>(a, p.d, nt, variant, num_items, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace li
