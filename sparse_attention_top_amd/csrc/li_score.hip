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
//   * 8 waves (two per SIMD, so one can issue while the other waits) = WQ rows x
//     WK key slices; a wave holds its row's query heads in AGPRs as MFMA
//     A-operands for the whole key loop;
//   * keys are staged KT at a time in LDS (double buffered through registers),
//     gathered through the block table for the paged layout;
//   * per 32-key slice a wave runs NT x (D / k-step) MFMA 32x32 ops with heads on
//     the M axis and keys on the N axis, with B fragments read one slice ahead;
//     each lane then holds 16 heads of one key per tile, applies ReLU and the
//     per-head weight (interleaved with the next slice's MFMAs), and one
//     cross-lane swap-add over the two half-waves completes the reduction.
#include "li_internal.h"

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

template <int DT, int D, int NT, int WQ, int WK, int KT>
__global__ __launch_bounds__(WQ * WK * 64) void score_kernel(ScoreArgs a) {
  using M = Mma<DT>;
  using Frag = typename M::Frag;
  using Acc = typename M::Acc;
  constexpr int ES = M::kElemBytes;
  constexpr int LB = M::kLaneBytes;
  constexpr int ROW = D * ES;              // bytes of one key row
  constexpr int KSTEPS = ROW / (2 * LB);   // MFMA k-steps over the head dim
  constexpr int ROWP = ROW + 16;           // LDS row pitch (16-byte pad vs bank conflicts)
  constexpr int NTHR = WQ * WK * 64;
  constexpr int CPR = ROW / 16;            // 16-byte chunks per key row
  constexpr int NCHUNK = KT * CPR;
  constexpr int CPT = (NCHUNK + NTHR - 1) / NTHR;
  constexpr bool QUANT = (DT == LI_DTYPE_E4M3FN) || (DT == LI_DTYPE_I8);
  constexpr int SPS = KT / 32 / WK;        // 32-key slices per staged tile per wave
  constexpr int EPM = 16 / KSTEPS;         // previous-slice accumulators per MFMA
  static_assert(KT % (32 * WK) == 0, "key tile must split into 32-key slices");
  static_assert(KSTEPS >= 1 && ROW % (2 * LB) == 0, "head dim must fill whole k-steps");
  static_assert(!QUANT || KT <= NTHR, "one thread per staged key scale");

  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][KT * ROWP];
  __shared__ float ksc[2][QUANT ? KT : 1];

  const WorkItem it = a.items[blockIdx.x];
  const BatchRec br = a.batches[it.b];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wq = wave % WQ;
  const int wk = wave / WQ;
  const int half = lane >> 5;
  const int col = lane & 31;

  const int row = it.q0 + wq;
  const bool row_ok = row < br.s_q;
  const int nv = row_ok ? visible_keys(row, br.s_q, br.s_k, a.sparse_mode) : 0;
  const int lim = nv < it.k1 ? nv : it.k1;   // this row stores keys [k0, lim)
  const int64_t qrow = (int64_t)br.row_base + (row_ok ? row : 0);
  float* out_row = a.ws + br.ws_off + (int64_t)(row_ok ? row : 0) * br.ld;

  // Query heads of this row as MFMA A-operands (zero for padded heads), and the
  // per-lane weights of the 16 heads each lane accumulates per tile.
  Frag qf[NT][KSTEPS];
  float wr[NT][16];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int h = 32 * t + col;
    const bool ok = row_ok && h < a.n1;
    const uint8_t* src = a.q + ((qrow * a.n1 + (ok ? h : 0)) * D) * ES + half * LB;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[t][s] = ok ? load_frag<Frag>(src + s * 2 * LB) : Frag{};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int he = 32 * t + 8 * (e >> 2) + 4 * half + (e & 3);
      float v = 0.f;
      if (row_ok && he < a.n1) {
        v = load_weight(a.w, a.dtype_w, qrow * a.n1 + he);
        if (QUANT) v *= a.q_scale[qrow * a.n1 + he];
      }
      wr[t][e] = v;
    }
  }

  // Global -> register prefetch of one key stage. Keys past k1 are clamped to
  // the last key of the item: their columns are computed but never stored, so
  // every load is unconditional (no per-lane branches, no zero fill).
  i32x4_t pre[CPT];
  float pre_sc = 0.f;
  const bool paged = a.layout_k == LI_LAYOUT_PA_BSND;
  const int jmax = it.k1 - 1;
  auto key_off = [&](int j) -> int64_t {   // element offset of key j's row
    if (paged) {
      int bi, bo;
      if (a.block_shift >= 0) {
        bi = j >> a.block_shift;
        bo = j & (a.block_size - 1);
      } else {
        bi = j / a.block_size;
        bo = j - bi * a.block_size;
      }
      int blk = a.block_table[(int64_t)it.b * a.max_blocks + bi];
      blk = blk < 0 ? 0 : (blk >= a.num_blocks ? (int)(a.num_blocks - 1) : blk);
      return (int64_t)blk * a.k_block_stride + (int64_t)bo * D;
    }
    return ((int64_t)br.k_base + j) * D;
  };
  auto scale_off = [&](int j) -> int64_t { // offset of key j's dequant scale
    if (paged) {
      int bi, bo;
      if (a.block_shift >= 0) {
        bi = j >> a.block_shift;
        bo = j & (a.block_size - 1);
      } else {
        bi = j / a.block_size;
        bo = j - bi * a.block_size;
      }
      int blk = a.block_table[(int64_t)it.b * a.max_blocks + bi];
      blk = blk < 0 ? 0 : (blk >= a.num_blocks ? (int)(a.num_blocks - 1) : blk);
      return (int64_t)blk * a.block_size + bo;
    }
    return (int64_t)br.k_base + j;
  };
  auto fetch = [&](int ks0) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = (tid + c * NTHR) % NCHUNK;   // NCHUNK < NTHR re-reads a chunk
      const int kk = ch / CPR;
      const int cc = ch - kk * CPR;
      const int j = min(ks0 + kk, jmax);
      pre[c] = *reinterpret_cast<const i32x4_t*>(a.k + key_off(j) * ES + cc * 16);
    }
    if (QUANT && tid < KT) pre_sc = a.k_scale[scale_off(min(ks0 + tid, jmax))];
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + c * NTHR;
      if (ch < NCHUNK) {
        const int kk = ch / CPR;
        const int cc = ch - kk * CPR;
        *reinterpret_cast<i32x4_t*>(&kbuf[buf][kk * ROWP + cc * 16]) = pre[c];
      }
    }
    if (QUANT && tid < KT) ksc[buf][tid] = pre_sc;
  };

  // Flat loop over this wave's 32-key slices. Every wave runs every slice of the
  // item (keys past a row's limit are computed but not stored), so barriers are
  // uniform. Slice g:
  //   * if g is the last slice of its staged tile: stash the next tile, barrier,
  //     start fetching the tile after it (so slice g+1's fragments can be read);
  //   * MFMAs of slice g; right after each k-step's MFMAs, that k-step's B
  //     fragment register is reloaded with slice g+1's (LDS latency hidden by a
  //     whole slice); the ReLU / weight / in-lane head reduction of slice g-1 is
  //     interleaved between the MFMAs;
  //   * cross-half swap-add and store of slice g-1.
  const int nstages = (it.k1 - it.k0 + KT - 1) / KT;
  const int nslices = nstages * SPS;
  fetch(it.k0);
  stash(0);
  __syncthreads();
  if (nstages > 1) fetch(it.k0 + KT);

  auto slice_loc = [&](int g, int& buf, int& sub) {
    const int st = g / SPS;
    sub = wk + (g - st * SPS) * WK;
    buf = st & 1;
    return it.k0 + st * KT + sub * 32;
  };
  auto boundary = [&](int g) {
    if ((g + 1) % SPS != 0) return;
    const int st = g / SPS;
    if (st + 1 < nstages) stash((st + 1) & 1);
    __syncthreads();
    if (st + 2 < nstages) fetch(it.k0 + (st + 2) * KT);
  };
  Frag bf[KSTEPS];
  {
    int buf, sub;
    slice_loc(0, buf, sub);
    const uint8_t* bsrc = &kbuf[buf][(sub * 32 + col) * ROWP + half * LB];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) bf[s] = load_frag<Frag>(bsrc + s * 2 * LB);
  }
  auto step = [&](int g, Acc (&acc)[NT], const Acc (&old)[NT], bool have_old, float& ks) {
    int buf, sub;
    slice_loc(g, buf, sub);
    ks = QUANT ? ksc[buf][sub * 32 + col] : 1.f;
    // Next slice's fragments (past the last slice: re-read this one, unused);
    // unconditional so that the MFMA / VALU block stays one basic block.
    int nbuf = buf, nsub = sub;
    if (g + 1 < nslices) slice_loc(g + 1, nbuf, nsub);
    const uint8_t* nsrc = &kbuf[nbuf][(nsub * 32 + col) * ROWP + half * LB];
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc[t] = M::mma(qf[t][s], bf[s], s == 0 ? M::zero() : acc[t]);
        if (have_old) {
#pragma unroll
          for (int u = 0; u < EPM; u += 2) {
            const int e = s * EPM + u;
            p0 = fmaf(wr[t][e], M::relu(old[t], e), p0);
            p1 = fmaf(wr[t][e + 1], M::relu(old[t], e + 1), p1);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      bf[s] = load_frag<Frag>(nsrc + s * 2 * LB);
    }
    return p0 + p1;
  };
  auto epi = [&](const Acc (&acc)[NT]) {
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        p0 = fmaf(wr[t][e], M::relu(acc[t], e), p0);
        p1 = fmaf(wr[t][e + 1], M::relu(acc[t], e + 1), p1);
      }
    }
    return p0 + p1;
  };
  // Cross-half swap-add (both halves end up with the full sum over heads) and
  // the store of the slice starting at key kb.
  auto finish = [&](float part, int kb, float ks) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part),
                                                     __float_as_uint(part), false, false);
    const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const int j = kb + col;
    if (half == 0 && j < lim) out_row[j] = QUANT ? tot * ks : tot;
  };
  auto key_of = [&](int g) {
    int buf, sub;
    return slice_loc(g, buf, sub);
  };

  Acc accA[NT], accB[NT];
  float ksA = 1.f, ksB = 1.f;
  boundary(0);
  step(0, accA, accB, false, ksA);
  int g = 1;
  for (; g + 1 < nslices; g += 2) {
    boundary(g);
    float part = step(g, accB, accA, true, ksB);
    finish(part, key_of(g - 1), ksA);
    boundary(g + 1);
    part = step(g + 1, accA, accB, true, ksA);
    finish(part, key_of(g), ksB);
  }
  if (g < nslices) {            // slice g computes into B, slice g-1 (A) drains
    boundary(g);
    const float part = step(g, accB, accA, true, ksB);
    finish(part, key_of(g - 1), ksA);
    finish(epi(accB), key_of(g), ksB);
  } else {
    finish(epi(accA), key_of(g - 1), ksA);
  }
}

template <int DT, int D, int NT>
hipError_t launch_v(int variant, int num_items, const ScoreArgs& a, hipStream_t s) {
  switch (variant) {
    case kVarPrefill:
      hipLaunchKernelGGL((score_kernel<DT, D, NT, 8, 1, 128>), dim3(num_items), dim3(512), 0, s, a);
      break;
    case kVarMid:
      hipLaunchKernelGGL((score_kernel<DT, D, NT, 4, 2, 128>), dim3(num_items), dim3(512), 0, s, a);
      break;
    case kVarDecode:
      hipLaunchKernelGGL((score_kernel<DT, D, NT, 2, 4, 128>), dim3(num_items), dim3(512), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(int d, int nt, int variant, int num_items, const ScoreArgs& a, hipStream_t s) {
  if (d == 128) return nt == 1 ? launch_v<DT, 128, 1>(variant, num_items, a, s)
                               : launch_v<DT, 128, 2>(variant, num_items, a, s);
  if (d == 64) return nt == 1 ? launch_v<DT, 64, 1>(variant, num_items, a, s)
                              : launch_v<DT, 64, 2>(variant, num_items, a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_score(const li_problem& p, int variant, int num_items, const ScoreArgs& a,
                        hipStream_t s) {
  if (num_items <= 0) return hipSuccess;
  const int nt = p.n1 > 32 ? 2 : 1;
  switch (p.dtype_qk) {
    case LI_DTYPE_BF16: return launch_dt<LI_DTYPE_BF16>(p.d, nt, variant, num_items, a, s);
    case LI_DTYPE_F16: return launch_dt<LI_DTYPE_F16>(p.d, nt, variant, num_items, a, s);
    case LI_DTYPE_E4M3FN: return launch_dt<LI_DTYPE_E4M3FN>(p.d, nt, variant, num_items, a, s);
    case LI_DTYPE_I8: return launch_dt<LI_DTYPE_I8>(p.d, nt, variant, num_items, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace li
