// Grouped SwiGLU expert MLP: one launch covers every local expert.
//
// Megatron Core MoE 源码路径解析 §10: the local experts' MLPs run as one
// grouped GEMM rather than a loop of small per-expert GEMMs.  Scalable
// Training of Mixture-of-Experts Models with Megatron Core (summary,
// 计算效率优化): grouped GEMM, and dropless routing executed without a
// host-device synchronisation on the per-expert token counts.
//
// Both GEMMs have the form C[m, n] = sum_k A[m, k] * B_e[n, k] with A the
// expert-major rows and B_e expert e's weight, both K-contiguous:
//   FC1: A = permuted_x [N, h], B = W_gate[e] and W_up[e] [f, h];
//        act = silu(gate) * up  (fused epilogue)
//   FC2: A = act [N, f], B = W_down[e] [h, f];  expert_out = A B^T
//
// Tile scheduler (no host sync): every workgroup reads tokens_per_expert,
// scans it in LDS (row offsets and M-tiles per expert), and decodes its own
// tile (expert, n-tile, m-tile) from its workgroup id.  The grid is sized on
// the host from the worst case (max_rows and E); surplus workgroups exit.
// Logical tile order is expert-major, then n-tile, then m-tile, so the
// m-tiles sharing one weight slab are adjacent; workgroup ids are remapped
// so that each of the 8 XCDs (which dispatch ids round-robin and own one L2
// each) runs a contiguous range of logical tiles.
//
// bf16 path: 8 waves per workgroup (two per SIMD); a tile body (the Body<>
// table near the launch code) is BM rows x BN weight rows per matrix, with
// one 32x32 block grid per wave and v_mfma_f32_32x32x16_bf16 accumulating in
// fp32.  The operands stream through a ring of 2-4 LDS stages of 64 k each,
// filled by direct global->LDS 16-byte loads (dma16) whose waits are
// counted explicitly: before the last 16-wide k step of stage kt every wave
// holds its fragments, the workgroup waits for stage kt+1 and passes one
// barrier, and stage kt's slot is refilled with stage kt+STAGES, the new
// loads issued one every SPREAD MFMAs.  LDS rows are 16-byte chunks
// XOR-swizzled (lds_chunk_byte in moe_internal.h) so that the direct loads
// fill contiguous 1 KB pieces and 16 lanes reading one chunk of 16 rows
// touch 16 different bank groups.  The weight fragment is the MFMA's first
// operand, so each lane ends with 4 consecutive output columns of one row
// (8-byte bf16 stores); FC1 holds gate and up accumulators for the same
// columns and applies silu(gate) * up in the epilogue.
//
// Launch variants: a 256-row launch picks the 256-, 128- or 64-row body per
// tile from its row count; single-expert launches take a grouped (banded)
// tile order; the shared expert's dense GEMM can ride as the last
// workgroups of a routed launch (DenseTail); given a tile queue, layers of
// experts with >= 192 rows on average run one workgroup per CU that takes
// tiles from per-XCD counters (the shared expert's tiles before the routed
// ones), their 256-row tiles on the split-ring body (gmm_tile_split:
// activation and weight rows in separate LDS rings, waves 0-3 issuing every
// load, waves 4-7 only multiplying); without one, layers of large, alike
// experts run one persistent workgroup per CU with a fixed tile sequence;
// top-1 layers can take the combine as FC2's epilogue.
#include <algorithm>
#include <type_traits>

#include "gmm_sched.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int BK = 64;


// ----------------------------------------------------------------- bf16 MFMA
// Pipeline schedules of a tile body (see gmm_tile).
constexpr int kSchedCompute = 0;
constexpr int kSchedRing = 1;

// MFMA operand fragments of one 16-wide k step for one wave: MI activation
// blocks and NB x NI weight blocks of 32 rows, 8 consecutive k per lane.
template <int MI, int NB, int NI, int BM, int BN, int SBK, int WTM, int WTN>
__device__ __forceinline__ void load_frags(bf16x8 (&a)[MI], bf16x8 (&b)[NB][NI], const char* st,
                                           int kk, int wm, int wn, int l32, int hi) {
  const int c = kk * 2 + hi;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int row = wm * WTM + mi * 32 + l32;
    a[mi] = *reinterpret_cast<const bf16x8*>(st + lds_chunk_byte<SBK>(row, c));
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int row = BM + nb * BN + wn * WTN + ni * 32 + l32;
      b[nb][ni] = *reinterpret_cast<const bf16x8*>(st + lds_chunk_byte<SBK>(row, c));
    }
}

template <int MI, int NB, int NI>
__device__ __forceinline__ void mfma_step(f32x16 (&acc)[NB][MI][NI], const bf16x8 (&a)[MI],
                                          const bf16x8 (&b)[NB][NI]) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[nb][mi][ni] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[nb][ni], a[mi], acc[nb][mi][ni], 0, 0, 0);
}

// Epilogue: lane holds C[m = l32][n = 8*g + 4*hi + q] of each 32x32 block;
// FC1 applies silu(gate) * up.  Rows >= nrows and columns >= N are not stored.
template <int MI, int NB, int NI, int WTM, int WTN, bool FC1>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[NB][MI][NI], uint16_t* __restrict__ C,
                                           int64_t row0, int nrows, int n0, int N, int wm, int wn,
                                           int l32, int hi) {
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int ml = wm * WTM + mi * 32 + l32;
    if (ml >= nrows) continue;
    uint16_t* crow = C + (row0 + ml) * static_cast<int64_t>(N);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WTN + ni * 32 + g * 8 + hi * 4;
        if (n >= N) continue;
        uint16_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v = FC1 ? silu_mul(acc[0][mi][ni][g * 4 + q], acc[NB - 1][mi][ni][g * 4 + q])
                              : acc[0][mi][ni][g * 4 + q];
          o[q] = f32_to_bf16_bits(v);
        }
        uint2 pk;
        pk.x = static_cast<uint32_t>(o[0]) | (static_cast<uint32_t>(o[1]) << 16);
        pk.y = static_cast<uint32_t>(o[2]) | (static_cast<uint32_t>(o[3]) << 16);
        *reinterpret_cast<uint2*>(crow + n) = pk;
      }
  }
}

template <int MI, int NI, int WTM, int WTN>
__device__ __forceinline__ void store_tile_combine(const f32x16 (&acc)[1][MI][NI],
                                                   const CombineEpi& epi, int64_t row0, int nrows,
                                                   int n0, int N, int wm, int wn, int l32, int hi) {
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int ml = wm * WTM + mi * 32 + l32;
    if (ml >= nrows) continue;
    const int64_t r = row0 + ml;
    int64_t t;
    if (!epi.owns(r, &t)) continue;
    const float p = epi.prob[r];
    uint16_t* crow = epi.out + t * static_cast<int64_t>(N);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WTN + ni * 32 + g * 8 + hi * 4;
        if (n >= N) continue;
        uint16_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = combine_bf16(p, acc[0][mi][ni][g * 4 + q]);
        uint2 pk;
        pk.x = static_cast<uint32_t>(o[0]) | (static_cast<uint32_t>(o[1]) << 16);
        pk.y = static_cast<uint32_t>(o[2]) | (static_cast<uint32_t>(o[3]) << 16);
        *reinterpret_cast<uint2*>(crow + n) = pk;
      }
  }
}

// LDS bytes one tile body uses.
template <int BM, int BN, bool FC1, int STAGES, int SBK>
constexpr int body_lds_bytes() {
  return STAGES * (BM + (FC1 ? 2 : 1) * BN) * SBK * 2;
}

// One output tile (BM rows of one expert x BN columns) of the grouped GEMM.
// `smem` holds the pipeline stages; all 64*WM*WN threads take part.
template <int BM, int BN, int WM, int WN, bool FC1, int STAGES, int SBK, int SCHED, int SPREAD,
          bool CMB>
__device__ __forceinline__ void gmm_tile(const Tile& tile, char* smem,
                                         const uint16_t* __restrict__ A,
                                         const int32_t* __restrict__ gather, int64_t a_rows,
                                         const uint16_t* __restrict__ B0,
                                         const uint16_t* __restrict__ B1, uint16_t* __restrict__ C,
                                         int N, int K, const CombineEpi& epi) {
  constexpr int NB = FC1 ? 2 : 1;
  constexpr int ROWS = BM + NB * BN;
  constexpr int NW = WM * WN;              // waves per workgroup
  constexpr int STAGE_BYTES = ROWS * SBK * 2;
  constexpr int LPW = STAGE_BYTES / (NW * 1024);  // direct loads (1 KB each) per wave per stage
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 32, NI = WTN / 32;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(MI >= 1 && NI >= 1, "wave tile must be at least 32x32");
  static_assert(STAGE_BYTES % (NW * 1024) == 0, "whole direct loads per wave");
  static_assert(SBK == 32 || SBK == 64 || SBK == 128 || SBK == 256, "k slab per stage");
  static_assert(SCHED == kSchedCompute || SCHED == kSchedRing, "schedule");
  static_assert((SCHED == kSchedRing && STAGES >= 2 && STAGES <= 6) ||
                    (SCHED == kSchedCompute && STAGES >= 3 && STAGES <= 6),
                "pipeline depth");

  const int n0 = tile.n0 * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const uint32_t smem_base = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));

  // Sources of this lane's direct loads (fixed rows; k advances per stage).
  // Rows past the tile's valid rows (or past N) are clamped in range: they
  // are computed but never stored.
  const uint16_t* src[LPW];
  const int64_t b_expert = static_cast<int64_t>(tile.e) * N * K;
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    int row, c;
    lds_piece<SBK>((wave * LPW + j) * 1024 + lane * 16, row, c);
    if (row < BM) {
      const int lr = min(row, tile.nrows - 1);
      int64_t ar = tile.row0 + lr;
      if (gather) ar = min(max(static_cast<int64_t>(gather[ar]), int64_t(0)), a_rows - 1);
      src[j] = A + ar * static_cast<int64_t>(K) + c * 8;
    } else {
      const int br = row - BM;
      const uint16_t* base = (NB == 2 && br >= BN) ? B1 : B0;
      const int n = min(n0 + (br % BN), N - 1);
      src[j] = base + b_expert + static_cast<int64_t>(n) * K + c * 8;
    }
  }
  auto issue = [&](int kt) {
    const uint32_t dst = smem_base + static_cast<uint32_t>((kt % STAGES) * STAGE_BYTES) +
                         static_cast<uint32_t>(wave * LPW * 1024);
    const int64_t ko = static_cast<int64_t>(kt) * SBK;
#pragma unroll
    for (int j = 0; j < LPW; ++j) dma16(src[j] + ko, dst + j * 1024);
  };

  f32x16 acc[NB][MI][NI];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[b][mi][ni][q] = 0.f;

  constexpr int KK = SBK / 16;
  const int nk = K / SBK;
  const int l32 = lane & 31, hi = lane >> 5;
  bf16x8 ca[MI], cb[NB][NI], na[MI], nb[NB][NI];
  if constexpr (SCHED == kSchedRing) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
      if (s < nk) issue(s);
  } else {
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < nk) issue(s);
  }
  if constexpr (SCHED == kSchedRing) {
    // Ring schedule: every slot holds a stage in flight or being multiplied.
    // Before the last 16-wide step of stage kt each wave has read all of
    // stage kt's fragments into registers (lgkmcnt 0); the workgroup waits
    // for stage kt+1 and passes a barrier, after which stage kt's slot
    // receives stage kt+STAGES and the first fragments of stage kt+1 are
    // read while the last MFMAs of stage kt run.  With SPREAD > 0 the new
    // stage's direct loads are not issued at once but one every SPREAD
    // MFMAs (counted from the barrier, so they continue into the first
    // steps of stage kt+1), so that a wave stalled on a full memory queue
    // still has MFMAs in flight.  The loop is split where the loads stop,
    // so that each iteration is straight-line code with constant waits (a
    // branch per load would split the block and let the compiler move the
    // MFMAs away from the loads placed between them).
    constexpr int MPK = NB * MI * NI;  // MFMAs per 16-wide step
    static_assert(SPREAD == 0 || LPW * SPREAD <= MPK * KK, "loads spread past the next barrier");
    auto piece = [&](int stage, int j) {
      const uint32_t dst = smem_base + static_cast<uint32_t>((stage % STAGES) * STAGE_BYTES) +
                           static_cast<uint32_t>(wave * LPW * 1024 + j * 1024);
      dma16(src[j] + static_cast<int64_t>(stage) * SBK, dst);
    };
    // one step's MFMAs; with ON, the pieces of `stage` due at MFMA
    // positions p0 .. p0+MPK-1 (counted from the barrier) are issued between them
    auto mfmas = [&](auto on_c, int p0, int stage) {
      constexpr bool ON = decltype(on_c)::value;
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            acc[q][mi][ni] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(cb[q][ni], ca[mi], acc[q][mi][ni], 0, 0, 0);
            if constexpr (ON) {
              const int pos = p0 + (q * MI + mi) * NI + ni;
              if (pos % SPREAD == 0 && pos / SPREAD < LPW) {
                piece(stage, pos / SPREAD);
                __builtin_amdgcn_sched_barrier(0);
              }
            }
          }
    };
    auto advance = [&]() {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) ca[mi] = na[mi];
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) cb[q][ni] = nb[q][ni];
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    // Stage kt.  PREV: stage kt-1+STAGES is being spread (issued from the
    // previous barrier on); CUR: stage kt+STAGES is issued at this one;
    // LAST: the final stage (no barrier).
    auto iter = [&](auto prev_c, auto cur_c, auto last_c, int kt) {
      constexpr bool PREV = decltype(prev_c)::value && SPREAD > 0;
      constexpr bool CUR = decltype(cur_c)::value, LAST = decltype(last_c)::value;
      const char* st = smem + (kt % STAGES) * STAGE_BYTES;
#pragma unroll
      for (int kk = 0; kk + 1 < KK; ++kk) {
        __builtin_amdgcn_sched_barrier(0);  // steps stay in order (bounded live fragments)
        load_frags<MI, NB, NI, BM, BN, SBK, WTM, WTN>(na, nb, st, kk + 1, wm, wn, l32, hi);
        mfmas(std::integral_constant<bool, PREV>{}, (kk + 1) * MPK, kt - 1 + STAGES);
        advance();
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!LAST) {
        // stage kt+1 has landed: at most the stages after it are in flight
        if constexpr (decltype(prev_c)::value || CUR) wait_vmcnt<(STAGES - 2) * LPW>();
        else wait_vmcnt<0>();
        wait_lgkm0();
        block_barrier();
        if constexpr (CUR && SPREAD == 0) issue(kt + STAGES);
        load_frags<MI, NB, NI, BM, BN, SBK, WTM, WTN>(
            na, nb, smem + ((kt + 1) % STAGES) * STAGE_BYTES, 0, wm, wn, l32, hi);
        mfmas(std::integral_constant<bool, CUR && (SPREAD > 0)>{}, 0, kt + STAGES);
        advance();
      } else {
        mfmas(F_{}, 0, 0);
      }
    };
    wait_stage<LPW, STAGES>(min(STAGES - 1, nk - 1));
    block_barrier();
    load_frags<MI, NB, NI, BM, BN, SBK, WTM, WTN>(ca, cb, smem, 0, wm, wn, l32, hi);
    int kt = 0;
    if (nk > 1) {
      if (STAGES < nk) iter(F_{}, T_{}, F_{}, 0);
      else iter(F_{}, F_{}, F_{}, 0);
      kt = 1;
    }
    for (; kt + STAGES < nk; ++kt) iter(T_{}, T_{}, F_{}, kt);
    if (kt >= 1 && kt + STAGES == nk && kt + 1 < nk) {  // its predecessor issued the last stage
      iter(T_{}, F_{}, F_{}, kt);
      ++kt;
    }
    for (; kt + 1 < nk; ++kt) iter(F_{}, F_{}, F_{}, kt);
    iter(F_{}, F_{}, T_{}, nk - 1);
    // the accumulators are complete here: keep the last MFMAs out of the
    // epilogue's conditional blocks
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) asm volatile("" : "+v"(acc[q][mi][ni]));
  } else {
    // Compute schedule (MFMA-bound bodies): stages kt+1 .. kt+STAGES-2 are
    // in flight while stage kt is multiplied; within a stage the fragments
    // of step kk+1 are read while the MFMAs of step kk run; before the last
    // step of stage kt the workgroup waits for stage kt+1, passes a barrier
    // (after which every wave is done with stage kt-1, whose slot then
    // receives stage kt+STAGES-1), and prefetches the first fragments of
    // stage kt+1.
    wait_stage<LPW, STAGES>(min(STAGES - 2, nk - 1));
    block_barrier();
    load_frags<MI, NB, NI, BM, BN, SBK, WTM, WTN>(ca, cb, smem, 0, wm, wn, l32, hi);
    for (int kt = 0; kt < nk; ++kt) {
      const char* st = smem + (kt % STAGES) * STAGE_BYTES;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) {
          load_frags<MI, NB, NI, BM, BN, SBK, WTM, WTN>(na, nb, st, kk + 1, wm, wn, l32, hi);
        } else if (kt + 1 < nk) {
          const int last = min(kt + STAGES - 2, nk - 1);  // newest stage issued so far
          wait_stage<LPW, STAGES>(last - (kt + 1));
          block_barrier();
          if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
          load_frags<MI, NB, NI, BM, BN, SBK, WTM, WTN>(
              na, nb, smem + ((kt + 1) % STAGES) * STAGE_BYTES, 0, wm, wn, l32, hi);
        }
        mfma_step<MI, NB, NI>(acc, ca, cb);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) ca[mi] = na[mi];
#pragma unroll
        for (int q = 0; q < NB; ++q)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) cb[q][ni] = nb[q][ni];
      }
    }
  }

  if constexpr (CMB && !FC1)
    store_tile_combine<MI, NI, WTM, WTN>(acc, epi, tile.row0, tile.nrows, n0, N, wm, wn, l32, hi);
  else
    store_tile<MI, NB, NI, WTM, WTN, FC1>(acc, C, tile.row0, tile.nrows, n0, N, wm, wn, l32, hi);
}


// --------------------------------------------- split-ring body (queue launches)
// The 256-row body of the tile-queue launches keeps the activation rows and
// the weight rows in rings of their own: 2 activation slots and 3 weight
// slots of 64 k (256 rows x 128 bytes each, 160 KB: all of LDS).  The weight
// rows, which stream from HBM, are issued two stages ahead of their use; the
// activation rows, which mostly hit L2, one stage ahead.  Waves 0-3 issue
// every direct load (eight activation and eight weight pieces of 1 KB per
// stage each) and waves 4-7 only multiply, so each SIMD holds one wave whose
// MFMAs never wait behind a load issue.  Sources are 32-bit byte offsets from
// a per-wave base in SGPRs (dma16s), sixteen of them in the registers that
// eight 64-bit pointers take.
constexpr int kSplitSlot = 256 * 128;
constexpr int kSplitLds = 5 * kSplitSlot;

template <int MI, int NB, int NI, int BN, int WTM, int WTN>
__device__ __forceinline__ void load_frags_split(bf16x8 (&a)[MI], bf16x8 (&b)[NB][NI],
                                                 const char* ast, const char* bst, int kk, int wm,
                                                 int wn, int l32, int hi) {
  const int c = kk * 2 + hi;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int row = wm * WTM + mi * 32 + l32;
    a[mi] = *reinterpret_cast<const bf16x8*>(ast + lds_chunk_byte<64>(row, c));
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int row = nb * BN + wn * WTN + ni * 32 + l32;
      b[nb][ni] = *reinterpret_cast<const bf16x8*>(bst + lds_chunk_byte<64>(row, c));
    }
}

// One 256-row tile (BN columns of W_gate and of W_up for FC1, BN = 128; of
// W_down for FC2, BN = 256).  Byte offsets of the activation rows must fit 31
// bits (a_rows * K * 2 <= 2^31), and so must those of one expert's weight
// rows (N * K * 2), and N must be a multiple of BN; the launcher checks all
// three.
//
// Schedule, per stage kt (64 k, four 16-wide steps): the first step's
// MFMAs carry the loaders' weight pieces of stage kt+2 (into the weight slot
// stage kt-1 released); before the last step each wave holds its fragments,
// the loaders wait until stage kt+1 has landed (the weight pieces of stage
// kt+2 may stay in flight), the workgroup passes one barrier, and the last
// step's MFMAs carry the activation pieces of stage kt+2 (into the slot
// stage kt released).  Loads of one loader complete in issue order, so the
// waits are counts of the pieces issued after the ones needed.
template <int BN, int WM, int WN, bool FC1>
__device__ __forceinline__ void gmm_tile_split(const Tile& tile, char* smem,
                                               const uint16_t* __restrict__ A,
                                               const int32_t* __restrict__ gather, int64_t a_rows,
                                               const uint16_t* __restrict__ B0,
                                               const uint16_t* __restrict__ B1,
                                               uint16_t* __restrict__ C, int N, int K) {
  constexpr int BM = 256, SBK = 64, KK = SBK / 16;
  constexpr int NB = FC1 ? 2 : 1;
  static_assert(NB * BN == 256, "256 weight rows per stage");
  static_assert(WM * WN == 8, "8 waves");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 32, NI = WTN / 32;
  static_assert(NB * MI * NI == 8, "8 MFMAs per 16-wide step: two pieces at every other one");
  const int n0 = tile.n0 * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, hi = lane >> 5;
  const uint32_t smem_base = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));
  const int nk = K / SBK;

  // Loader w (waves 0-3) fills pieces 8w .. 8w+7 of each block: rows 64w ..
  // 64w+63 of the activation rows and of the weight rows (FC1: w < 2 reads
  // W_gate, w >= 2 W_up).  Rows past the tile's rows (or past N) are clamped
  // in range: they are computed but never stored.
  const bool loader = wave < 4;
  const int w = loader ? wave : 0;
  const char* abase = uniform_ptr(A);
  const char* bbase =
      uniform_ptr((FC1 && w >= 2 ? B1 : B0) + static_cast<int64_t>(tile.e) * N * K);
  // Weight piece j holds rows 8 (8w + j) + lane / 8, i.e. weight rows
  // n0 + 64 (w % 2) + 8 j + lane / 8 (FC1) or n0 + 64 w + 8 j + lane / 8
  // (FC2), all below N (N is a multiple of BN): a lane's pieces step by 8
  // rows (folded into the base) and their 16-byte chunk depends on j's
  // parity only (lds_piece's swizzle), so two offsets serve all eight.
  uint32_t aoff[8], boff[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int row, c;
    lds_piece<SBK>((8 * w + j) * 1024 + lane * 16, row, c);
    int64_t ar = tile.row0 + min(row, tile.nrows - 1);
    if (gather) ar = min(max(static_cast<int64_t>(gather[ar]), int64_t(0)), a_rows - 1);
    aoff[j] = static_cast<uint32_t>(ar * K * 2 + c * 16);
    if (j < 2) {
      const int n = n0 + row % BN;
      boff[j] = static_cast<uint32_t>(static_cast<int64_t>(n) * K * 2 + c * 16);
    }
  }
  auto slot_a = [&](int s) { return (s & 1) * kSplitSlot; };
  auto slot_b = [&](int s) { return (2 + s % 3) * kSplitSlot; };
  auto piece_a = [&](int s, int j) {
    dma16s(aoff[j], abase + s * (SBK * 2), smem_base + slot_a(s) + (8 * w + j) * 1024);
  };
  auto piece_b = [&](int s, int j) {
    dma16s(boff[j & 1], bbase + s * (SBK * 2) + static_cast<int64_t>(j & ~1) * 8 * K * 2,
           smem_base + slot_b(s) + (8 * w + j) * 1024);
  };

  f32x16 acc[NB][MI][NI];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[b][mi][ni][q] = 0.f;
  bf16x8 ca[MI], cb[NB][NI], na[MI], nb[NB][NI];

  // prologue: activation and weight pieces of stages 0 and 1, weights of
  // stage 2 (those that exist), in that order; then stage 0 must be in
  if (loader) {
#pragma unroll
    for (int j = 0; j < 8; ++j) piece_a(0, j);
#pragma unroll
    for (int j = 0; j < 8; ++j) piece_b(0, j);
    if (nk > 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) piece_a(1, j);
#pragma unroll
      for (int j = 0; j < 8; ++j) piece_b(1, j);
    }
    if (nk > 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j) piece_b(2, j);
      wait_vmcnt<24>();
    } else if (nk > 1) {
      wait_vmcnt<16>();
    } else {
      wait_vmcnt<0>();
    }
  }
  block_barrier();
  load_frags_split<MI, NB, NI, BN, WTM, WTN>(ca, cb, smem, smem + slot_b(0), 0, wm, wn, l32, hi);

  // one step's MFMAs; with IA (IB) the loader's eight activation (weight)
  // pieces of stage s go out two at every other MFMA
  auto mfmas = [&](auto ia_c, auto ib_c, int s) {
    constexpr bool IA = decltype(ia_c)::value, IB = decltype(ib_c)::value;
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          acc[q][mi][ni] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(cb[q][ni], ca[mi], acc[q][mi][ni], 0, 0, 0);
          if constexpr (IA || IB) {
            const int pos = (q * MI + mi) * NI + ni;
            if (pos % 2 == 0) {
              if constexpr (IA) {
                piece_a(s, pos);
                piece_a(s, pos + 1);
              } else {
                piece_b(s, pos);
                piece_b(s, pos + 1);
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
  };
  auto advance = [&]() {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) ca[mi] = na[mi];
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) cb[q][ni] = nb[q][ni];
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  // Stage kt.  LD: this wave is a loader; IB0: its first step issues the
  // weight pieces of stage kt+2; IA3: its last step the activation pieces of
  // stage kt+2; W8: the wait before the barrier leaves those weight pieces
  // in flight; LAST: the final stage (no barrier).
  auto iter = [&](auto ld_c, auto ib0_c, auto ia3_c, auto w8_c, auto last_c, int kt) {
    constexpr bool LD = decltype(ld_c)::value;
    constexpr bool IB0 = LD && decltype(ib0_c)::value, IA3 = LD && decltype(ia3_c)::value;
    constexpr bool W8 = decltype(w8_c)::value, LAST = decltype(last_c)::value;
    const char* ast = smem + slot_a(kt);
    const char* bst = smem + slot_b(kt);
#pragma unroll
    for (int kk = 0; kk + 1 < KK; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      load_frags_split<MI, NB, NI, BN, WTM, WTN>(na, nb, ast, bst, kk + 1, wm, wn, l32, hi);
      if (kk == 0) mfmas(F_{}, std::integral_constant<bool, IB0>{}, kt + 2);
      else mfmas(F_{}, F_{}, 0);
      advance();
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!LAST) {
      if constexpr (LD) {
        if constexpr (W8) wait_vmcnt<8>();
        else wait_vmcnt<0>();
      }
      wait_lgkm0();
      block_barrier();
      load_frags_split<MI, NB, NI, BN, WTM, WTN>(na, nb, smem + slot_a(kt + 1),
                                                 smem + slot_b(kt + 1), 0, wm, wn, l32, hi);
      mfmas(std::integral_constant<bool, IA3>{}, F_{}, kt + 2);
      advance();
    } else {
      mfmas(F_{}, F_{}, 0);
    }
  };
  auto run = [&](auto ld) {
    if (nk == 1) {
      iter(ld, F_{}, F_{}, F_{}, T_{}, 0);
      return;
    }
    if (nk >= 3) iter(ld, F_{}, T_{}, T_{}, F_{}, 0);  // stage 2's weights came with the prologue
    else iter(ld, F_{}, F_{}, F_{}, F_{}, 0);
    int kt = 1;
    for (; kt + 2 < nk; ++kt) iter(ld, T_{}, T_{}, T_{}, F_{}, kt);
    if (kt == nk - 2) {
      iter(ld, F_{}, F_{}, F_{}, F_{}, kt);
      ++kt;
    }
    iter(ld, F_{}, F_{}, F_{}, T_{}, kt);
  };
  if (loader) run(T_{});
  else run(F_{});
  // the accumulators are complete here: keep the last MFMAs out of the
  // epilogue's conditional blocks
#pragma unroll
  for (int q = 0; q < NB; ++q)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) asm volatile("" : "+v"(acc[q][mi][ni]));
  store_tile<MI, NB, NI, WTM, WTN, FC1>(acc, C, tile.row0, tile.nrows, n0, N, wm, wn, l32, hi);
}

// The grouped-GEMM kernel: decode this workgroup's tile with BMAX-row
// m-tiles, then run a tile body.  With 256-row m-tiles an expert's last,
// ragged tile runs the 128- or 64-row body when it fits (less MFMA work
// spent on padding); with shorter m-tiles the layer is weight-streaming
// bound and one body serves every tile.  The choice is uniform per
// workgroup.
// A dense GEMM run by the last `wgs` workgroups of a grouped launch (the
// shared expert: all tokens through one weight, [MC] §11), so that its tiles
// fill the tail of the routed experts' tiles in one launch.  Grouped tile
// order as dense_tile_at; A rows are not gathered.
struct DenseTail {
  const uint16_t* A;
  const uint16_t* B0;
  const uint16_t* B1;
  uint16_t* C;
  int64_t rows;
  int N, K;
  int wgs;
};

template <bool FC1, int BMAX, int BN, int NW, class Body256, class Body128, class Body64,
          bool CMB = false, bool DENSE = false, bool TAIL = false, bool PERSIST = false,
          bool QUEUE = false>
__global__ void __launch_bounds__(NW * 64) gmm_bf16_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ gather, int64_t a_rows,
    const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1,
    uint16_t* __restrict__ C, const int32_t* __restrict__ counts, int E, int N, int K,
    int64_t max_rows, CombineEpi epi, const int32_t* __restrict__ row_id_map, int zero_wgs,
    DenseTail dn, int* __restrict__ queue) {
  if constexpr (CMB) {
    const int z = static_cast<int>(blockIdx.x) - static_cast<int>(gridDim.x - zero_wgs);
    if (z >= 0) {  // the last workgroups zero the dropped tokens (in the tail of the tiles)
      zero_dropped_rows(row_id_map, max_rows, epi.out, epi.T, N, z);
      return;
    }
  }
  constexpr int L256 = Body256::lds > Body128::lds ? Body256::lds : Body128::lds;
  constexpr int LDS = BMAX == 256 ? (L256 > Body64::lds ? L256 : Body64::lds)
                                 : (BMAX == 128 ? Body128::lds : Body64::lds);
  constexpr int DECODE_BYTES = (3 * kMaxExperts + 1) * 4 + 64;
  static_assert(LDS >= DECODE_BYTES, "decode scratch aliases the stages");
  __shared__ __attribute__((aligned(1024))) char smem[LDS];
  if constexpr (QUEUE) {
    // One workgroup per CU takes tiles from the queue (queue_tiles): the
    // dense tail's logical tiles, then the routed experts' (kDenseFirst).
    const int NT = (N + BN - 1) / BN;
    __shared__ int p_toff[kPersistMaxExperts + 1], p_roff[kPersistMaxExperts],
        p_n[kPersistMaxExperts];
    __shared__ int s_kq;
    decode_to_tables<BMAX, NW * 64>(counts, E, max_rows, smem, p_toff, p_roff, p_n);
    const int64_t routed = static_cast<int64_t>(p_toff[E]) * NT;
    const int ntd = TAIL ? (dn.N + BN - 1) / BN : 0;
    const int64_t total = routed + (TAIL ? (dn.rows + BMAX - 1) / BMAX * ntd : 0);
    // Once its own XCD's tiles run out, a workgroup takes the remaining
    // tiles of the other XCDs, one XCD after another (a counter only grows,
    // so an XCD found empty stays empty): the XCDs end together.  (The same
    // loop as queue_tiles, written out: through the lambda the FC2 kernels
    // spilled two registers.)
    const int x = static_cast<int>(blockIdx.x % 8);
    for (int v = 0; v < 8;) {
      const int xv = (x + v) % 8;
      if (threadIdx.x == 0) s_kq = atomicAdd(queue + xv * kQStride, 1);
      __syncthreads();
      const int64_t kq = s_kq;
      __syncthreads();  // s_kq is rewritten by the next take
      const int64_t L = ((kq / kQGroup) * 8 + xv) * kQGroup + kq % kQGroup;
      if (kq < 0 || L >= total) {  // uniform over the workgroup
        ++v;
        continue;
      }
      Tile t;
      const uint16_t* ta = A;
      const int32_t* tg = gather;
      int64_t tar = a_rows;
      const uint16_t* tb0 = B0;
      const uint16_t* tb1 = B1;
      uint16_t* tc = C;
      int tn = N, tk = K;
      const int64_t nd = total - routed;  // the dense tail's tiles
      if (TAIL && (kDenseFirst ? L < nd : L >= routed)) {
        t = dense_tile_at<BMAX, kDenseBand>(kDenseFirst ? L : L - routed, ntd, dn.rows, 0);
        ta = dn.A;
        tg = nullptr;
        tar = dn.rows;
        tb0 = dn.B0;
        tb1 = dn.B1;
        tc = dn.C;
        tn = dn.N;
        tk = dn.K;
      } else {
        t = tile_at<BMAX>(TAIL && kDenseFirst ? L - nd : L, NT, E, p_toff, p_roff, p_n);
      }
      t.nrows = __builtin_amdgcn_readfirstlane(t.nrows);
      if (t.nrows > 128) Body256::template run<CMB>(t, smem, ta, tg, tar, tb0, tb1, tc, tn, tk, epi);
      else if (t.nrows > 64) Body128::template run<CMB>(t, smem, ta, tg, tar, tb0, tb1, tc, tn, tk, epi);
      else Body64::template run<CMB>(t, smem, ta, tg, tar, tb0, tb1, tc, tn, tk, epi);
      __syncthreads();  // every wave is past the tile before its stages are refilled
    }
    queue_leave(queue);
    return;
  }
  // this workgroup's tile and its operands (the routed experts', or the
  // dense tail's), then one call of the body its row count selects
  Tile tile;
  const uint16_t* a = A;
  const int32_t* g = gather;
  int64_t ar = a_rows;
  const uint16_t* b0 = B0;
  const uint16_t* b1 = B1;
  uint16_t* c = C;
  int n = N, k = K;
  bool mine;
  // the tail starts at a multiple of 8, so d % 8 is this workgroup's XCD
  const int d = TAIL ? static_cast<int>(blockIdx.x) - static_cast<int>(gridDim.x - dn.wgs) : -1;
  if (TAIL && d >= 0) {
    const int ntd = (dn.N + BN - 1) / BN;
    const int64_t L = xcd_tile(d, (dn.rows + BMAX - 1) / BMAX * ntd);
    mine = L >= 0;
    if (mine) tile = dense_tile_at<BMAX, kDenseBand>(L, ntd, dn.rows, 0);
    a = dn.A;
    g = nullptr;
    ar = dn.rows;
    b0 = dn.B0;
    b1 = dn.B1;
    c = dn.C;
    n = dn.N;
    k = dn.K;
  } else if constexpr (PERSIST) {
    // One workgroup per CU runs tiles b, b + grid, b + 2 grid, ... of the
    // XCD-ordered sequence (grid a multiple of 8, so each keeps its XCD):
    // at each step the workgroups of an XCD hold consecutive tiles, as a
    // one-tile-per-workgroup grid would, but the counts are decoded once
    // and no workgroup is launched per tile.  Used where experts are
    // large and alike in size (the tiles take about equal time, so the
    // fixed assignment stays balanced).
    const int NT = (N + BN - 1) / BN;
    __shared__ int p_toff[kPersistMaxExperts + 1], p_roff[kPersistMaxExperts],
        p_n[kPersistMaxExperts];
    decode_to_tables<BMAX, NW * 64>(counts, E, max_rows, smem, p_toff, p_roff, p_n);
    const int64_t total = static_cast<int64_t>(p_toff[E]) * NT;
    for (int64_t j = blockIdx.x;; j += gridDim.x) {
      const int64_t L = xcd_tile(j, total);
      if (L < 0) return;  // uniform: every wave of the workgroup leaves here
      Tile t = tile_at<BMAX>(L, NT, E, p_toff, p_roff, p_n);
      t.nrows = __builtin_amdgcn_readfirstlane(t.nrows);
      if constexpr (BMAX == 256) {
        if (t.nrows > 128) Body256::template run<CMB>(t, smem, a, g, ar, b0, b1, c, n, k, epi);
        else if (t.nrows > 64) Body128::template run<CMB>(t, smem, a, g, ar, b0, b1, c, n, k, epi);
        else Body64::template run<CMB>(t, smem, a, g, ar, b0, b1, c, n, k, epi);
      } else if constexpr (BMAX == 128) {
        Body128::template run<CMB>(t, smem, a, g, ar, b0, b1, c, n, k, epi);
      } else {
        Body64::template run<CMB>(t, smem, a, g, ar, b0, b1, c, n, k, epi);
      }
      __syncthreads();  // every wave is past the tile before its stages are refilled
    }
  } else {
    const int NT = (N + BN - 1) / BN;
    int* s_toff = reinterpret_cast<int*>(smem);
    int* s_roff = s_toff + kMaxExperts + 1;
    int* s_n = s_roff + kMaxExperts;
    int64_t* s_scan = reinterpret_cast<int64_t*>(s_n + kMaxExperts + 1);
    mine = DENSE ? decode_dense_tile<BMAX, kDenseBand>(counts, max_rows, NT, s_n, tile)
                 : decode_tile<BMAX, NW * 64>(counts, E, max_rows, NT, s_toff, s_roff, s_n, s_scan,
                                              tile);
    __syncthreads();  // decode scratch is reused by the stages below
  }
  if (!mine) return;
  tile.nrows = __builtin_amdgcn_readfirstlane(tile.nrows);
  if constexpr (BMAX == 256) {
    if (tile.nrows > 128) Body256::template run<CMB>(tile, smem, a, g, ar, b0, b1, c, n, k, epi);
    else if (tile.nrows > 64) Body128::template run<CMB>(tile, smem, a, g, ar, b0, b1, c, n, k, epi);
    else Body64::template run<CMB>(tile, smem, a, g, ar, b0, b1, c, n, k, epi);
  } else if constexpr (BMAX == 128) {
    Body128::template run<CMB>(tile, smem, a, g, ar, b0, b1, c, n, k, epi);
  } else {
    Body64::template run<CMB>(tile, smem, a, g, ar, b0, b1, c, n, k, epi);
  }
}

// Tile-queue launch with the split-ring 256-row body (gmm_tile_split): one
// workgroup per CU takes tiles from the queue as queue_tiles does.  The
// stages take all of LDS, so no decoded tables are kept: for each tile the
// first wave decodes the counts again (WaveCounts, E <= kPersistMaxExperts)
// and hands the tile to the others through the first bytes of LDS.  Ragged
// tiles of <= 128 rows run the 128- and 64-row bodies of the plain queue
// launch; the shared expert's tiles (DenseTail) come before the routed ones
// (kDenseFirst).
template <bool FC1, int BN, int WM, int WN, class Body128, class Body64, bool TAIL>
__global__ void __launch_bounds__(512) gmm_bf16_qsplit_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ gather, int64_t a_rows,
    const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, uint16_t* __restrict__ C,
    const int32_t* __restrict__ counts, int E, int N, int K, int64_t max_rows, DenseTail dn,
    int* __restrict__ queue) {
  static_assert(Body128::lds <= kSplitLds && Body64::lds <= kSplitLds, "bodies fit the stages");
  __shared__ __attribute__((aligned(1024))) char smem[kSplitLds];
  int* hdr = reinterpret_cast<int*>(smem);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int NT = (N + BN - 1) / BN;
  const int ntd = TAIL ? (dn.N + BN - 1) / BN : 0;
  const int64_t dense = TAIL ? (dn.rows + 255) / 256 * ntd : 0;
  const int x = static_cast<int>(blockIdx.x % 8);
  int v = 0;  // XCDs drained so far (first wave)
  for (;;) {
    if (wave == 0) {
      WaveCounts wc;
      int64_t L = -1;
      if constexpr (!FC1) {
        // the take is issued before the counts load, so that their latencies
        // overlap (FC2's short tiles gain 2.5-5 %; kept out of FC1, whose
        // launch was measured slower with it)
        int take = 0;
        if (v < 8 && lane == 0) take = atomicAdd(queue + ((x + v) % 8) * kQStride, 1);
        wc.load<256>(counts, E, max_rows);
        const int64_t total = static_cast<int64_t>(wc.mtiles) * NT + dense;
        while (v < 8) {  // its XCD's next tile, then the other XCDs' remaining ones
          const int xv = (x + v) % 8;
          const int kq = __builtin_amdgcn_readlane(take, 0);
          const int64_t Lc =
              (static_cast<int64_t>(kq / kQGroup) * 8 + xv) * kQGroup + kq % kQGroup;
          if (kq >= 0 && Lc < total) {
            L = Lc;
            break;
          }
          if (++v < 8 && lane == 0) take = atomicAdd(queue + ((x + v) % 8) * kQStride, 1);
        }
      } else {
        wc.load<256>(counts, E, max_rows);
        const int64_t total = static_cast<int64_t>(wc.mtiles) * NT + dense;
        while (v < 8) {  // its XCD's next tile, then the other XCDs' remaining ones
          const int xv = (x + v) % 8;
          int kq = 0;
          if (lane == 0) kq = atomicAdd(queue + xv * kQStride, 1);
          kq = __shfl(kq, 0, 64);
          const int64_t Lc =
              (static_cast<int64_t>(kq / kQGroup) * 8 + xv) * kQGroup + kq % kQGroup;
          if (kq >= 0 && Lc < total) {
            L = Lc;
            break;
          }
          ++v;
        }
      }
      const int64_t routed = static_cast<int64_t>(wc.mtiles) * NT;
      Tile t{0, 0, 0, 0};
      int src = -1;  // -1: none left; 0: routed; 1: dense tail
      if (L >= 0) {
        if (TAIL && (kDenseFirst ? L < dense : L >= routed)) {
          t = dense_tile_at<256, kDenseBand>(kDenseFirst ? L : L - routed, ntd, dn.rows, 0);
          src = 1;
        } else {
          t = wc.tile<256>(TAIL && kDenseFirst ? L - dense : L, NT, E);
          src = 0;
        }
      }
      if (lane == 0) {
        hdr[0] = src;
        hdr[1] = t.e;
        hdr[2] = static_cast<int>(static_cast<uint32_t>(t.row0));
        hdr[3] = static_cast<int>(static_cast<uint64_t>(t.row0) >> 32);
        hdr[4] = t.nrows;
        hdr[5] = t.n0;
      }
    }
    __syncthreads();
    const int src = __builtin_amdgcn_readfirstlane(hdr[0]);
    Tile t;
    t.e = __builtin_amdgcn_readfirstlane(hdr[1]);
    t.row0 = static_cast<int64_t>(
        (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(hdr[3]))) << 32) |
        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(hdr[2])));
    t.nrows = __builtin_amdgcn_readfirstlane(hdr[4]);
    t.n0 = __builtin_amdgcn_readfirstlane(hdr[5]);
    __syncthreads();  // the header's bytes belong to the tile's first stage
    if (src < 0) break;
    const bool dn_tile = TAIL && src == 1;
    const uint16_t* ta = dn_tile ? dn.A : A;
    const int32_t* tg = dn_tile ? nullptr : gather;
    const int64_t tar = dn_tile ? dn.rows : a_rows;
    const uint16_t* tb0 = dn_tile ? dn.B0 : B0;
    const uint16_t* tb1 = dn_tile ? dn.B1 : B1;
    uint16_t* tc = dn_tile ? dn.C : C;
    const int tn = dn_tile ? dn.N : N, tk = dn_tile ? dn.K : K;
    const CombineEpi no_epi{nullptr, nullptr, nullptr, 0, nullptr};
    if (t.nrows > 128) gmm_tile_split<BN, WM, WN, FC1>(t, smem, ta, tg, tar, tb0, tb1, tc, tn, tk);
    else if (t.nrows > 64) Body128::template run<false>(t, smem, ta, tg, tar, tb0, tb1, tc, tn, tk, no_epi);
    else Body64::template run<false>(t, smem, ta, tg, tar, tb0, tb1, tc, tn, tk, no_epi);
    __syncthreads();  // every wave is past the tile before its stages are refilled
  }
  queue_leave(queue);
}

template <int BM, int BN, int WM, int WN, bool FC1, int STAGES, int SBK, int SCHED = kSchedCompute,
          int SPREAD = 0>
struct Body {
  static constexpr int lds = body_lds_bytes<BM, BN, FC1, STAGES, SBK>();
  template <bool CMB>
  __device__ __forceinline__ static void run(const Tile& t, char* smem, const uint16_t* A,
                                             const int32_t* gather, int64_t a_rows,
                                             const uint16_t* B0, const uint16_t* B1, uint16_t* C,
                                             int N, int K, const CombineEpi& epi) {
    gmm_tile<BM, BN, WM, WN, FC1, STAGES, SBK, SCHED, SPREAD, CMB>(t, smem, A, gather, a_rows, B0,
                                                                   B1, C, N, K, epi);
  }
};

// ----------------------------------------------------------------- fp32 MFMA
// For fp32 layers: 64x64 tiles (per weight matrix) on the fp32 matrix
// cores, v_mfma_f32_32x32x2_f32: four waves, each owning a 32x32 block of
// the tile, multiply k-slabs of 16 staged through LDS (k-major, so lane l of
// a wave reads row l % 32 of its block at k = 2s + l / 32 without bank
// conflicts); any N and K (the slab past K is zero-filled).  Every product
// and sum is fp32, as in the layer's fp32 arithmetic; the order of the
// k-sums differs from a sequential loop by rounding only.
constexpr int FM = 64, FN = 64, FK = 16;

template <bool FC1>
__global__ void __launch_bounds__(kThreads) gmm_f32_kernel(const float* __restrict__ A,
                                                           const int32_t* __restrict__ gather,
                                                           int64_t a_rows,
                                                           const float* __restrict__ B0,
                                                           const float* __restrict__ B1,
                                                           float* __restrict__ C,
                                                           const int32_t* __restrict__ counts,
                                                           int E, int N, int K, int64_t max_rows) {
  constexpr int NB = FC1 ? 2 : 1;
  static_assert(kThreads == 256, "four waves, one 32x32 block each");
  __shared__ float as[FK][FM + 4];
  __shared__ float bs[NB][FK][FN + 4];
  __shared__ int s_toff[kMaxExperts + 1];
  __shared__ int s_roff[kMaxExperts];
  __shared__ int s_n[kMaxExperts];
  __shared__ int64_t s_scan[8];
  const int NT = (N + FN - 1) / FN;
  Tile tile;
  if (!decode_tile<FM>(counts, E, max_rows, NT, s_toff, s_roff, s_n, s_scan, tile)) return;
  const int n0 = tile.n0 * FN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
  f32x16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[b][q] = 0.f;
  for (int k0 = 0; k0 < K; k0 += FK) {
    for (int i = tid; i < FM * FK; i += kThreads) {
      const int rr = i / FK, kk = i % FK;
      const int k = k0 + kk;
      const int lr = min(rr, tile.nrows - 1);
      int64_t ar = tile.row0 + lr;
      if (gather) ar = min(max(static_cast<int64_t>(gather[ar]), int64_t(0)), a_rows - 1);
      as[kk][rr] = k < K ? A[ar * static_cast<int64_t>(K) + k] : 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float* B = b == 0 ? B0 : B1;
        const int n = min(n0 + rr, N - 1);
        bs[b][kk][rr] = k < K ? B[(static_cast<int64_t>(tile.e) * N + n) * K + k] : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < FK / 2; ++s) {
      // weights as the first operand: lane l then holds output row
      // (token) l % 32 and columns 8 g + 4 (l / 32) + q in acc[4 g + q]
      const float av = as[2 * s + hi][wm * 32 + l32];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(bs[b][2 * s + hi][wn * 32 + l32], av, acc[b],
                                                      0, 0, 0);
    }
    __syncthreads();
  }
  const int ml = wm * 32 + l32;
  if (ml >= tile.nrows) return;
  float* crow = C + (tile.row0 + ml) * static_cast<int64_t>(N);
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + wn * 32 + g * 8 + hi * 4 + q;
      if (n >= N) continue;
      crow[n] = FC1 ? silu_mul(acc[0][g * 4 + q], acc[NB - 1][g * 4 + q]) : acc[0][g * 4 + q];
    }
}

// ----------------------------------------------------------------- launch

// The activation operand: row i of the grouped GEMM is row gather[i] of
// `base` (rows in [0, rows)) when `gather` is given, else row i.
struct AOperand {
  const void* base;
  const int32_t* gather;
  int64_t rows;
};

// With a combine epilogue (cmb.epi.out set), ceil(T / (16 * waves))
// workgroups after the tile workgroups zero the dropped tokens' rows (they
// are dispatched last, onto CUs the last round of tiles leaves idle).
struct CombineArgs {
  CombineEpi epi{nullptr, nullptr, nullptr, 0, nullptr};
  const int32_t* row_id_map = nullptr;
};

// The shared expert's dense GEMM, run in the same launch (see DenseTail).
struct SharedArgs {
  const void* A = nullptr;  // [rows, K]
  const void* B0 = nullptr;
  const void* B1 = nullptr;
  void* C = nullptr;  // [rows, N]
  int64_t rows = 0, N = 0, K = 0;
};

template <bool FC1, int BMAX, int BN, int NW, class B256, class B128, class B64,
          bool PERSIST = false, bool QUEUE = false>
void launch_bf16(const AOperand& a, const void* B0, const void* B1, void* C, const int32_t* counts,
                 int64_t E, int64_t N, int64_t K, int64_t max_rows, hipStream_t s,
                 const CombineArgs& cmb = CombineArgs{}, const SharedArgs& sh = SharedArgs{},
                 int* queue = nullptr) {
  const int64_t g = grid_for(max_rows, E, BMAX, N, BN);
  const int64_t z = cmb.epi.out ? ceil_div(cmb.epi.T, NW * 16) : 0;
  DenseTail dn{static_cast<const uint16_t*>(sh.A), static_cast<const uint16_t*>(sh.B0),
               static_cast<const uint16_t*>(sh.B1), static_cast<uint16_t*>(sh.C), sh.rows,
               static_cast<int>(sh.N), static_cast<int>(sh.K), 0};
  if (sh.rows > 0) dn.wgs = static_cast<int>(grid_for(sh.rows, 1, BMAX, sh.N, BN));
  const auto args = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(g + z + dn.wgs)), dim3(NW * 64), 0, s,
                       static_cast<const uint16_t*>(a.base), a.gather, a.rows,
                       static_cast<const uint16_t*>(B0), static_cast<const uint16_t*>(B1),
                       static_cast<uint16_t*>(C), counts, static_cast<int>(E), static_cast<int>(N),
                       static_cast<int>(K), max_rows, cmb.epi, cmb.row_id_map, static_cast<int>(z),
                       dn, static_cast<int*>(nullptr));
  };
  if constexpr (QUEUE) {  // callers pass a queue and exclude the combine epilogue
    if (g + dn.wgs == 0) return;
    const auto k = dn.wgs > 0
                       ? gmm_bf16_kernel<FC1, BMAX, BN, NW, B256, B128, B64, false, false, true, false, true>
                       : gmm_bf16_kernel<FC1, BMAX, BN, NW, B256, B128, B64, false, false, false, false, true>;
    hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(persistent_grid(g + dn.wgs))), dim3(NW * 64), 0,
                       s, static_cast<const uint16_t*>(a.base), a.gather, a.rows,
                       static_cast<const uint16_t*>(B0), static_cast<const uint16_t*>(B1),
                       static_cast<uint16_t*>(C), counts, static_cast<int>(E), static_cast<int>(N),
                       static_cast<int>(K), max_rows, cmb.epi, cmb.row_id_map, 0, dn, queue);
    return;
  }
  if (dn.wgs > 0) {  // routed tiles, then the shared expert's (never with the combine epilogue)
    args(gmm_bf16_kernel<FC1, BMAX, BN, NW, B256, B128, B64, false, false, true>);
    return;
  }
  if constexpr (PERSIST) {  // callers exclude the combine epilogue and the shared tail
    if (g == 0) return;
    hipLaunchKernelGGL((gmm_bf16_kernel<FC1, BMAX, BN, NW, B256, B128, B64, false, false, false, true>),
                       dim3(static_cast<unsigned>(persistent_grid(g))), dim3(NW * 64), 0, s,
                       static_cast<const uint16_t*>(a.base), a.gather, a.rows,
                       static_cast<const uint16_t*>(B0), static_cast<const uint16_t*>(B1),
                       static_cast<uint16_t*>(C), counts, static_cast<int>(E), static_cast<int>(N),
                       static_cast<int>(K), max_rows, cmb.epi, cmb.row_id_map, 0, dn,
                       static_cast<int*>(nullptr));
    return;
  }
  if constexpr (!FC1 && (BMAX != 256 || BN == 128)) {  // (the combine epilogue's launches)
    if (cmb.epi.out) {
      args(gmm_bf16_kernel<FC1, BMAX, BN, NW, B256, B128, B64, true>);
      return;
    }
  }
  if (E == 1) {  // one dense GEMM (the shared expert): grouped tile order
    args(gmm_bf16_kernel<FC1, BMAX, BN, NW, B256, B128, B64, false, true>);
    return;
  }
  args(gmm_bf16_kernel<FC1, BMAX, BN, NW, B256, B128, B64, false>);
}

// The split-ring queue launch (gmm_bf16_qsplit_kernel) takes 32-bit source
// offsets: every activation row and every expert's weight rows must lie
// within 2^31 bytes of their base; and its n-tiles must be whole (N a
// multiple of the tile width BN).
bool split_fits(const AOperand& a, int64_t N, int64_t K, int BN, const SharedArgs& sh) {
  const int64_t lim = int64_t(1) << 31;
  if (a.rows * K * 2 > lim || N * K * 2 > lim || N % BN != 0) return false;
  return sh.rows == 0 || (sh.rows * sh.K * 2 <= lim && sh.N * sh.K * 2 <= lim && sh.N % BN == 0);
}

template <bool FC1, int BN, int WM, int WN, class B128, class B64>
void launch_qsplit(const AOperand& a, const void* B0, const void* B1, void* C,
                   const int32_t* counts, int64_t E, int64_t N, int64_t K, int64_t max_rows,
                   hipStream_t s, const SharedArgs& sh, int* queue) {
  const int64_t g = grid_for(max_rows, E, 256, N, BN);
  DenseTail dn{static_cast<const uint16_t*>(sh.A), static_cast<const uint16_t*>(sh.B0),
               static_cast<const uint16_t*>(sh.B1), static_cast<uint16_t*>(sh.C), sh.rows,
               static_cast<int>(sh.N), static_cast<int>(sh.K), 0};
  if (sh.rows > 0) dn.wgs = static_cast<int>(grid_for(sh.rows, 1, 256, sh.N, BN));
  if (g + dn.wgs == 0) return;
  const auto k = dn.wgs > 0 ? gmm_bf16_qsplit_kernel<FC1, BN, WM, WN, B128, B64, true>
                            : gmm_bf16_qsplit_kernel<FC1, BN, WM, WN, B128, B64, false>;
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(persistent_grid(g + dn.wgs))), dim3(512), 0, s,
                     static_cast<const uint16_t*>(a.base), a.gather, a.rows,
                     static_cast<const uint16_t*>(B0), static_cast<const uint16_t*>(B1),
                     static_cast<uint16_t*>(C), counts, static_cast<int>(E), static_cast<int>(N),
                     static_cast<int>(K), max_rows, dn, queue);
}

template <bool FC1>
void launch_f32(const AOperand& a, const void* B0, const void* B1, void* C, const int32_t* counts,
                int64_t E, int64_t N, int64_t K, int64_t max_rows, hipStream_t s) {
  const int64_t g = grid_for(max_rows, E, FM, N, FN);
  hipLaunchKernelGGL((gmm_f32_kernel<FC1>), dim3(static_cast<unsigned>(g)), dim3(kThreads), 0, s,
                     static_cast<const float*>(a.base), a.gather, a.rows,
                     static_cast<const float*>(B0), static_cast<const float*>(B1),
                     static_cast<float*>(C), counts, static_cast<int>(E), static_cast<int>(N),
                     static_cast<int>(K), max_rows);
}

// Tile shape from the average rows per expert (known on the host without
// reading the device counts): tall tiles amortise weight reads when experts
// are large; shorter tiles waste fewer MFMA cycles on padding when they are
// not.  All variants run 8 waves (two per SIMD, so one wave's MFMAs cover
// the other's waits); the shapes were chosen by timing the variants on the
// five layer shapes.
// 256-row m-tiles from 128 rows per expert on: an expert with 129-256 rows
// is then one tile (the 256-row body) instead of a full tile and a short
// one that streams the same weight slab again (timed on the Switch layer
// with capacity 160: FC1 440 vs 445 us, FC2 with the combine 234 vs 246 us).
int pick_bm(int64_t max_rows, int64_t E) {
  const int64_t avg = max_rows / E;
  if (avg >= 128) return 256;
  if (avg >= 80) return 128;
  return 64;
}

// Tile bodies (8 waves each; shapes chosen by timing variants on the five
// layer shapes with random operands).  All bodies of one launch share the
// column tiling.  256-row launches: FC1 tiles hold BN=128 columns of
// W_gate and of W_up; FC2 tiles 256 columns of W_down from 192 rows per
// expert on (MFMA-bound), else 128 (weight-streaming bound; also the
// bodies of the combine epilogue); ragged tails run 128- or 64-row
// bodies.  128- and 64-row launches (small experts, weight-streaming
// bound) use one body each.
using Fc1B256 = Body<256, 128, 2, 4, true, 2, 64, kSchedRing, 2>;
using Fc1B128 = Body<128, 128, 2, 4, true, 3, 64, kSchedRing, 2>;
using Fc1B64 = Body<64, 128, 2, 4, true, 4, 64>;
using Fc2B256 = Body<256, 256, 4, 2, false, 2, 64, kSchedRing, 2>;
using Fc2B128 = Body<128, 256, 2, 4, false, 3, 64, kSchedRing, 2>;
using Fc2B64 = Body<64, 256, 2, 4, false, 4, 64>;
using Fc2B128n = Body<128, 128, 2, 4, false, 4, 64, kSchedRing, 1>;  // 128-row launches
using Fc2N256 = Body<256, 128, 2, 4, false, 3, 64, kSchedRing, 2>;    // 256 rows, 128 columns
using Fc2N64 = Body<64, 128, 2, 4, false, 4, 64>;
// 64-row bodies of persistent launches: 3 stages, leaving LDS for the
// decoded per-expert tables
using Fc1B64p = Body<64, 128, 2, 4, true, 3, 64>;
using Fc2B64p = Body<64, 256, 2, 4, false, 3, 64>;
// 64-row bodies of the split-ring queue launches, which keep no tables in
// LDS: 4 stages (160 KB), three in flight for these weight-streaming tiles
using Fc1B64q = Body<64, 128, 2, 4, true, 4, 64>;
using Fc2B64q = Body<64, 256, 2, 4, false, 4, 64>;

// Persistent launches (see gmm_bf16_kernel) for experts of >= 512 rows on
// average, at most kPersistMaxExperts of them: measured on the Mixtral- and
// Qwen3-shaped layers FC1 -3 to -4 %, FC2 -5 to -10 %.  With smaller,
// unevenly sized experts (the DeepSeek-V3-shaped layer, 1..836 rows) the
// fixed tile assignment lets workgroups drift apart and lose their shared
// L2 lines (FC1 +17 %), so those keep one tile per workgroup, which the
// dispatcher hands out in order.
bool use_persistent(int64_t max_rows, int64_t E) {
  return E > 1 && E <= kPersistMaxExperts && max_rows / E >= 512;
}

// Tile-queue launches (a queue given): from 192 rows per expert on average.
// Measured against one workgroup per tile: DeepSeek-V3-shaped FC1 5.76 ->
// 5.46 ms and FC2 3.16 -> 2.89 ms in the layer (no idle gaps between tiles,
// XCDs finishing together); Mixtral-shaped FC2 -10 %, Qwen3-shaped FC1
// -4.5 % and FC2 -6 %.  Launches of small experts only stream weights, and
// there the queue lost 6 % (the Switch-shaped FC1, 160 rows per expert), so
// they keep one workgroup per tile.
bool use_queue(int64_t max_rows, int64_t E) {
  return E > 1 && E <= kPersistMaxExperts && max_rows / E >= 192;
}

template <bool FC1>
void launch_gemm(int32_t dtype, const AOperand& A, const void* B0, const void* B1, void* C,
                 const int32_t* counts, int64_t E, int64_t N, int64_t K, int64_t max_rows,
                 hipStream_t s, const CombineArgs& cmb = CombineArgs{},
                 const SharedArgs& sh = SharedArgs{}, void* queue = nullptr) {
  if (dtype == MOE_F32) {
    launch_f32<FC1>(A, B0, B1, C, counts, E, N, K, max_rows, s);
    return;
  }
  const int bm = pick_bm(max_rows, E);
  int* q = static_cast<int*>(queue);
  if (q && use_queue(max_rows, E) && !cmb.epi.out) {  // tile-queue launch (bm == 256 here)
    if (split_fits(A, N, K, FC1 ? 128 : 256, sh)) {
      if constexpr (FC1)
        launch_qsplit<true, 128, 2, 4, Fc1B128, Fc1B64q>(A, B0, B1, C, counts, E, N, K, max_rows, s, sh, q);
      else
        launch_qsplit<false, 256, 4, 2, Fc2B128, Fc2B64q>(A, B0, B1, C, counts, E, N, K, max_rows, s, sh, q);
      return;
    }
    if constexpr (FC1)
      launch_bf16<true, 256, 128, 8, Fc1B256, Fc1B128, Fc1B64p, false, true>(A, B0, B1, C, counts, E, N, K, max_rows, s, cmb, sh, q);
    else
      launch_bf16<false, 256, 256, 8, Fc2B256, Fc2B128, Fc2B64p, false, true>(A, B0, B1, C, counts, E, N, K, max_rows, s, cmb, sh, q);
    return;
  }
  if (!cmb.epi.out && sh.rows == 0 && use_persistent(max_rows, E)) {  // bm == 256 here
    if constexpr (FC1)
      launch_bf16<true, 256, 128, 8, Fc1B256, Fc1B128, Fc1B64p, true>(A, B0, B1, C, counts, E, N, K, max_rows, s);
    else
      launch_bf16<false, 256, 256, 8, Fc2B256, Fc2B128, Fc2B64p, true>(A, B0, B1, C, counts, E, N, K, max_rows, s);
    return;
  }
  if constexpr (FC1) {
    if (bm == 256)
      launch_bf16<true, 256, 128, 8, Fc1B256, Fc1B128, Fc1B64>(A, B0, B1, C, counts, E, N, K, max_rows, s, cmb, sh);
    else if (bm == 128)
      launch_bf16<true, 128, 128, 8, Fc1B128, Fc1B128, Fc1B128>(A, B0, B1, C, counts, E, N, K, max_rows, s, cmb, sh);
    else
      launch_bf16<true, 64, 128, 8, Fc1B64, Fc1B64, Fc1B64>(A, B0, B1, C, counts, E, N, K, max_rows, s, cmb, sh);
  } else {
    if (bm == 256 && max_rows / E >= 192 && !cmb.epi.out)
      launch_bf16<false, 256, 256, 8, Fc2B256, Fc2B128, Fc2B64>(A, B0, B1, C, counts, E, N, K, max_rows, s, cmb, sh);
    else if (bm == 256)
      launch_bf16<false, 256, 128, 8, Fc2N256, Fc2B128n, Fc2N64>(A, B0, B1, C, counts, E, N, K, max_rows, s, cmb, sh);
    else if (bm == 128)
      launch_bf16<false, 128, 128, 8, Fc2B128n, Fc2B128n, Fc2B128n>(A, B0, B1, C, counts, E, N, K, max_rows, s, cmb, sh);
    else
      launch_bf16<false, 64, 256, 8, Fc2B64, Fc2B64, Fc2B64>(A, B0, B1, C, counts, E, N, K, max_rows, s, cmb, sh);
  }
}

moe_status validate(const char* who, int64_t E, int64_t h, int64_t f, int64_t max_rows,
                    int32_t dtype) {
  MOE_REQUIRE(E >= 1 && E <= kMaxExperts, MOE_ERR_ARG, "%s: E=%lld not in [1,%lld]", who,
              (long long)E, (long long)kMaxExperts);
  MOE_REQUIRE(h >= 1 && f >= 1, MOE_ERR_ARG, "%s: h and f must be positive", who);
  MOE_REQUIRE(max_rows >= 0 && max_rows < (int64_t(1) << 31), MOE_ERR_ARG,
              "%s: max_rows out of range", who);
  MOE_REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, MOE_ERR_ARG, "%s: bad dtype %d", who, dtype);
  MOE_REQUIRE(E * f < (int64_t(1) << 31) && E * h < (int64_t(1) << 31) &&
                  h * f < (int64_t(1) << 31),
              MOE_ERR_UNSUPPORTED, "%s: E*f, E*h or h*f too large", who);
  if (dtype == MOE_BF16)
    MOE_REQUIRE(h % BK == 0 && f % BK == 0, MOE_ERR_UNSUPPORTED,
                "%s: bf16 needs h and f to be multiples of %d (h=%lld f=%lld)", who, BK,
                (long long)h, (long long)f);
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_grouped_fc1_swiglu(int64_t E, int64_t h, int64_t f, int64_t max_rows,
                                             int32_t dtype, const void* permuted_x,
                                             const int32_t* tokens_per_expert, const void* w_gate,
                                             const void* w_up, void* act, void* queue, void* stream) {
  moe_status st = validate("moe_grouped_fc1_swiglu", E, h, f, max_rows, dtype);
  if (st != MOE_OK) return st;
  if (max_rows == 0) return MOE_OK;
  MOE_REQUIRE(permuted_x && tokens_per_expert && w_gate && w_up && act, MOE_ERR_ARG,
              "moe_grouped_fc1_swiglu: NULL tensor argument");
  launch_gemm<true>(dtype, AOperand{permuted_x, nullptr, max_rows}, w_gate, w_up, act,
                    tokens_per_expert, E, f, h, max_rows, as_stream(stream), CombineArgs{},
                    SharedArgs{}, queue);
  return check_launch("moe_grouped_fc1_swiglu");
}

extern "C" moe_status moe_grouped_fc1_swiglu_gather(int64_t E, int64_t h, int64_t f,
                                                    int64_t max_rows, int32_t dtype, int64_t T,
                                                    const void* x, const int32_t* sorted_token,
                                                    const int32_t* tokens_per_expert,
                                                    const void* w_gate, const void* w_up, void* act,
                                                    void* queue, void* stream) {
  moe_status st = validate("moe_grouped_fc1_swiglu_gather", E, h, f, max_rows, dtype);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(T >= 0 && T < (int64_t(1) << 31), MOE_ERR_ARG,
              "moe_grouped_fc1_swiglu_gather: T out of range");
  if (max_rows == 0 || T == 0) return MOE_OK;
  MOE_REQUIRE(x && sorted_token && tokens_per_expert && w_gate && w_up && act, MOE_ERR_ARG,
              "moe_grouped_fc1_swiglu_gather: NULL tensor argument");
  launch_gemm<true>(dtype, AOperand{x, sorted_token, T}, w_gate, w_up, act, tokens_per_expert, E,
                    f, h, max_rows, as_stream(stream), CombineArgs{}, SharedArgs{}, queue);
  return check_launch("moe_grouped_fc1_swiglu_gather");
}

extern "C" moe_status moe_grouped_fc1_swiglu_gather_shared(
    int64_t E, int64_t h, int64_t f, int64_t max_rows, int32_t dtype, int64_t T, const void* x,
    const int32_t* sorted_token, const int32_t* tokens_per_expert, const void* w_gate,
    const void* w_up, void* act, int64_t fs, const void* shared_gate, const void* shared_up,
    void* shared_act, void* queue, void* stream) {
  const char* who = "moe_grouped_fc1_swiglu_gather_shared";
  moe_status st = validate(who, E, h, f, max_rows, dtype);
  if (st != MOE_OK) return st;
  st = validate(who, 1, h, fs, T, dtype);  // the shared expert: one expert of T rows
  if (st != MOE_OK) return st;
  MOE_REQUIRE(T >= 0 && T < (int64_t(1) << 31), MOE_ERR_ARG, "%s: T out of range", who);
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(x && shared_gate && shared_up && shared_act, MOE_ERR_ARG, "%s: NULL tensor argument",
              who);
  MOE_REQUIRE(max_rows == 0 || (sorted_token && tokens_per_expert && w_gate && w_up && act),
              MOE_ERR_ARG, "%s: NULL tensor argument", who);
  MOE_REQUIRE(dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "%s: bf16 only", who);
  const hipStream_t s = as_stream(stream);
  SharedArgs sh;
  sh.A = x;
  sh.B0 = shared_gate;
  sh.B1 = shared_up;
  sh.C = shared_act;
  sh.rows = T;
  sh.N = fs;
  sh.K = h;
  launch_gemm<true>(dtype, AOperand{x, sorted_token, T}, w_gate, w_up, act, tokens_per_expert, E, f,
                    h, max_rows, s, CombineArgs{}, sh, queue);
  return check_launch(who);
}

extern "C" moe_status moe_grouped_fc2(int64_t E, int64_t h, int64_t f, int64_t max_rows,
                                      int32_t dtype, const void* act,
                                      const int32_t* tokens_per_expert, const void* w_down,
                                      void* expert_out, void* queue, void* stream) {
  moe_status st = validate("moe_grouped_fc2", E, h, f, max_rows, dtype);
  if (st != MOE_OK) return st;
  if (max_rows == 0) return MOE_OK;
  MOE_REQUIRE(act && tokens_per_expert && w_down && expert_out, MOE_ERR_ARG,
              "moe_grouped_fc2: NULL tensor argument");
  launch_gemm<false>(dtype, AOperand{act, nullptr, max_rows}, w_down, nullptr, expert_out,
                     tokens_per_expert, E, h, f, max_rows, as_stream(stream), CombineArgs{},
                     SharedArgs{}, queue);
  return check_launch("moe_grouped_fc2");
}

extern "C" moe_status moe_grouped_fc2_shared(int64_t E, int64_t h, int64_t f, int64_t max_rows,
                                             int32_t dtype, const void* act,
                                             const int32_t* tokens_per_expert, const void* w_down,
                                             void* expert_out, int64_t T, int64_t fs,
                                             const void* shared_act, const void* shared_down,
                                             void* shared_out, void* queue, void* stream) {
  const char* who = "moe_grouped_fc2_shared";
  moe_status st = validate(who, E, h, f, max_rows, dtype);
  if (st != MOE_OK) return st;
  st = validate(who, 1, h, fs, T, dtype);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(T >= 0 && T < (int64_t(1) << 31), MOE_ERR_ARG, "%s: T out of range", who);
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(shared_act && shared_down && shared_out, MOE_ERR_ARG, "%s: NULL tensor argument",
              who);
  MOE_REQUIRE(max_rows == 0 || (act && tokens_per_expert && w_down && expert_out), MOE_ERR_ARG,
              "%s: NULL tensor argument", who);
  MOE_REQUIRE(dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "%s: bf16 only", who);
  const hipStream_t s = as_stream(stream);
  SharedArgs sh;
  sh.A = shared_act;
  sh.B0 = shared_down;
  sh.C = shared_out;
  sh.rows = T;
  sh.N = h;
  sh.K = fs;
  launch_gemm<false>(dtype, AOperand{act, nullptr, max_rows}, w_down, nullptr, expert_out,
                     tokens_per_expert, E, h, f, max_rows, s, CombineArgs{}, sh, queue);
  return check_launch(who);
}

extern "C" moe_status moe_grouped_fc2_combine(int64_t E, int64_t h, int64_t f, int64_t max_rows,
                                              int32_t dtype, int64_t T, const void* act,
                                              const int32_t* tokens_per_expert, const void* w_down,
                                              const float* permuted_probs,
                                              const int32_t* sorted_token,
                                              const int32_t* row_id_map, void* out, void* stream) {
  moe_status st = validate("moe_grouped_fc2_combine", E, h, f, max_rows, dtype);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(dtype == MOE_BF16, MOE_ERR_UNSUPPORTED, "moe_grouped_fc2_combine: bf16 only");
  MOE_REQUIRE(T >= 0 && T < (int64_t(1) << 31), MOE_ERR_ARG,
              "moe_grouped_fc2_combine: T out of range");
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(row_id_map && out && tokens_per_expert && w_down, MOE_ERR_ARG,
              "moe_grouped_fc2_combine: NULL tensor argument");
  MOE_REQUIRE(max_rows == 0 || (act && permuted_probs && sorted_token), MOE_ERR_ARG,
              "moe_grouped_fc2_combine: NULL tensor argument");
  CombineArgs cmb;
  cmb.epi = CombineEpi{sorted_token, permuted_probs, static_cast<uint16_t*>(out), T, row_id_map};
  cmb.row_id_map = row_id_map;
  launch_gemm<false>(dtype, AOperand{act, nullptr, max_rows}, w_down, nullptr, nullptr,
                     tokens_per_expert, E, h, f, max_rows, as_stream(stream), cmb);
  return check_launch("moe_grouped_fc2_combine");
}

extern "C" moe_status moe_grouped_mlp(int64_t E, int64_t h, int64_t f, int64_t max_rows,
                                      int32_t dtype, const void* permuted_x,
                                      const int32_t* tokens_per_expert, const void* w_gate,
                                      const void* w_up, const void* w_down, void* act,
                                      void* expert_out, void* queue, void* stream) {
  moe_status st = moe_grouped_fc1_swiglu(E, h, f, max_rows, dtype, permuted_x, tokens_per_expert,
                                         w_gate, w_up, act, queue, stream);
  if (st != MOE_OK) return st;
  return moe_grouped_fc2(E, h, f, max_rows, dtype, act, tokens_per_expert, w_down, expert_out,
                         queue, stream);
}
