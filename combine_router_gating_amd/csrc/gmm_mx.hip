// Grouped SwiGLU expert MLP on MXFP8 operands (gfx950 scaled MFMA).
//
// Scalable Training of Mixture-of-Experts Models with Megatron Core (FP8/FP4
// 低精度训练, 计算效率优化): FP8 GEMMs in the grouped expert MLP.  Operands are
// MXFP8-E4M3 (mx.hip): every 32 consecutive values along the reduction
// dimension share an E8M0 scale.  v_mfma_scale_f32_32x32x64_f8f6f4 takes 32
// E4M3 values per lane and applies both operands' block scales itself: lane
// l supplies row l%32; its bytes 0-15 are 16 values of the step's first
// 32-value block and bytes 16-31 16 values of the second, the two lane halves
// splitting each block, and lane l's scale register holds the scale of block
// l/32 of its row (checked on the hardware against a host evaluation).
//
//   FC1: act = silu(x Wg^T) * (x Wu^T) in fp32, quantised to MXFP8 along f in
//        the epilogue (a row's 32-column block lives in two lanes, lane l and
//        l^32, so its largest magnitude takes one exchange);
//   FC2: expert_out = act Wd^T, stored bf16.
// The tile scheduler is the bf16 GEMM's (gmm_sched.h); a stage holds 128 k
// (128 bytes per row, the same swizzled LDS layout) plus the rows' 4 scale
// bytes, all filled by direct global->LDS loads.  Tile-queue launches run the
// split-ring body (mx_tile_split) as the bf16 GEMM's do, and their ragged
// tiles of at most 64 rows a 64-row body.
#include <type_traits>

#include "gmm_sched.h"
#include "mx_codec.h"

namespace moe {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMxK = 128;  // k per stage: 128 E4M3 bytes per row, 4 scale bytes

// acc += (b with scale sb) x (a with scale sa), fenced.  The scaled fp8
// MFMA reads its 8-register operands over several cycles after it issues;
// the compiler's hazard model does not cover that, and a value it placed in
// a dead operand register right after the MFMA was seen to corrupt the
// product.  So no instruction of this wave issues for 16 wait states after
// it (the scheduling barriers keep the window next to the MFMA).
__device__ __forceinline__ void mx_mfma(f32x16& acc, const i32x8& b, const i32x8& a, int sb, int sa) {
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc, 0, 0, 0, sb, 0, sa);
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

struct MxA {
  const uint8_t* codes;    // [a_rows, K]
  const uint8_t* scales;   // row-major [a_rows, K/32], or k-tiled [K/128, a_rows, 4]
  const int32_t* gather;   // GEMM row i reads source row gather[i], or row i if NULL
  int64_t rows;            // a_rows
  bool tiled;              // scale layout
};
struct MxB {
  const uint8_t* codes0;   // [E, N, K]
  const uint8_t* scales0;  // k-tiled [E, K/128, N, 4]
  const uint8_t* codes1;   // FC1: W_up
  const uint8_t* scales1;
};
struct MxOut {
  uint8_t* codes;      // FC1: act codes [max_rows, N]
  uint8_t* scales;     // FC1: act scales, k-tiled [N/128, max_rows, 4]
  uint16_t* bf16;      // FC2: expert_out [max_rows, N]
  int64_t rows;        // max_rows
  CombineEpi cmb{nullptr, nullptr, nullptr, 0, nullptr};  // FC2 with the top-1 combine: out [T, N]
  const int32_t* row_id_map = nullptr;           // [T] (dropped tokens' zero rows)
};

template <int BM, int BN, bool FC1, int NW, int STAGES>
constexpr int mx_lds_bytes() {
  return STAGES * ((BM + (FC1 ? 2 : 1) * BN) * kMxK + NW * 64 * 4);
}

// Epilogue of an MXFP8 tile: lane holds C[m = l32][n = 8g + 4*hi + q] of
// each 32x32 block.  FC1: act = silu(gate) * up quantised to MXFP8 along f;
// FC2: bf16 expert_out, or with CMB the top-1 combine into out.
template <int MI, int NB, int NI, int WTM, int WTN, bool FC1, bool CMB>
__device__ __forceinline__ void mx_store(const f32x16 (&acc)[NB][MI][NI], const Tile& tile,
                                         const MxOut& O, int N, int n0, int wm, int wn, int l32,
                                         int hi) {
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int ml = wm * WTM + mi * 32 + l32;
    const bool row_ok = ml < tile.nrows;
    const int64_t grow = tile.row0 + ml;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int nc = n0 + wn * WTN + ni * 32;  // first column of this 32-column block
      if constexpr (FC1) {
        float v[16];
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float g = acc[0][mi][ni][i], u = acc[1][mi][ni][i];
          v[i] = g / (1.0f + __expf(-g)) * u;
          amax = fmaxf(amax, fabsf(v[i]));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));  // the row's other 16 columns
        const int e = mx_scale_exp(amax);
        const float inv = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
        if (row_ok && nc < N) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint32_t word = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) word |= e4m3_code(v[4 * g + q] * inv) << (8 * q);
            *reinterpret_cast<uint32_t*>(O.codes + grow * N + nc + 8 * g + 4 * hi) = word;
          }
          if (hi == 0)
            O.scales[((nc / kMxK) * O.rows + grow) * 4 + ((nc / 32) & 3)] = static_cast<uint8_t>(e + 127);
        }
      } else if constexpr (CMB) {
        int64_t t;
        if (!row_ok || nc >= N || !O.cmb.owns(grow, &t)) continue;
        const float p = O.cmb.prob[grow];
        uint16_t* crow = O.cmb.out + t * N;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint2 pk;
          pk.x = static_cast<uint32_t>(combine_bf16(p, acc[0][mi][ni][4 * g])) |
                 (static_cast<uint32_t>(combine_bf16(p, acc[0][mi][ni][4 * g + 1])) << 16);
          pk.y = static_cast<uint32_t>(combine_bf16(p, acc[0][mi][ni][4 * g + 2])) |
                 (static_cast<uint32_t>(combine_bf16(p, acc[0][mi][ni][4 * g + 3])) << 16);
          *reinterpret_cast<uint2*>(crow + nc + 8 * g + 4 * hi) = pk;
        }
      } else {
        if (!row_ok || nc >= N) continue;
        uint16_t* crow = O.bf16 + grow * N;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint2 pk;
          pk.x = static_cast<uint32_t>(f32_to_bf16_bits(acc[0][mi][ni][4 * g])) |
                 (static_cast<uint32_t>(f32_to_bf16_bits(acc[0][mi][ni][4 * g + 1])) << 16);
          pk.y = static_cast<uint32_t>(f32_to_bf16_bits(acc[0][mi][ni][4 * g + 2])) |
                 (static_cast<uint32_t>(f32_to_bf16_bits(acc[0][mi][ni][4 * g + 3])) << 16);
          *reinterpret_cast<uint2*>(crow + nc + 8 * g + 4 * hi) = pk;
        }
      }
    }
  }
}

// One output tile (BM rows of one expert x BN columns).
template <int BM, int BN, int WM, int WN, bool FC1, int STAGES, int SPREAD, bool CMB>
__device__ __forceinline__ void mx_tile(const Tile& tile, char* smem, const MxA& A, const MxB& B,
                                        const MxOut& O, int N, int K) {
  constexpr int NB = FC1 ? 2 : 1;
  constexpr int ROWS = BM + NB * BN;
  constexpr int NW = WM * WN;
  constexpr int DATA = ROWS * kMxK;
  constexpr int STAGE_BYTES = DATA + NW * 64 * 4;
  constexpr int LPW = DATA / (NW * 1024);  // 1 KB data loads per wave per stage
  constexpr int LPWT = LPW + 1;            // plus one 256-byte scale load
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 32, NI = WTN / 32;
  static_assert(DATA % (NW * 1024) == 0, "whole data loads per wave");
  static_assert(NW * 64 >= ROWS, "one scale row per lane");
  static_assert(MI >= 1 && NI >= 1, "wave tile at least 32x32");
  static_assert(STAGES >= 2 && STAGES <= 4, "pipeline depth");

  const int n0 = tile.n0 * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, hi = lane >> 5;
  const uint32_t smem_base = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));
  const int64_t KB = K / 32;  // scale bytes per row (row-major layout)
  const int nk = K / kMxK;    // stages
  const int64_t b_expert = static_cast<int64_t>(tile.e) * N;

  // source row (clamped in range; padding rows are computed, never stored)
  auto a_row = [&](int r) {
    int64_t ar = tile.row0 + min(r, tile.nrows - 1);
    if (A.gather) ar = min(max(static_cast<int64_t>(A.gather[ar]), int64_t(0)), A.rows - 1);
    return ar;
  };
  // A 1 KB piece covers 8 whole LDS rows, and BM and BN are multiples of 64,
  // so whether a piece (or a wave's scale row) belongs to A, W0 or W1 is the
  // same in every lane: the branches below are uniform.
  const uint8_t* src[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int prow0 = (wave * LPW + j) * 8;  // first LDS row of the piece
    int row, c;
    lds_piece<64>((wave * LPW + j) * 1024 + lane * 16, row, c);
    if (prow0 < BM) {
      src[j] = A.codes + a_row(row) * K + c * 16;
    } else {
      const int br = row - BM;
      const uint8_t* base = (NB == 2 && prow0 - BM >= BN) ? B.codes1 : B.codes0;
      const int n = min(n0 + (br % BN), N - 1);
      src[j] = base + (b_expert + n) * K + c * 16;
    }
  }
  // this lane's scale dword of stage kt: ssrc + kt * sstep (k-tiled layouts
  // put consecutive rows next to each other, so a wave's loads coalesce)
  const uint8_t* ssrc;
  int64_t sstep;
  {
    const int r = min(wave * 64 + lane, ROWS - 1);
    if (wave * 64 < BM) {
      const int64_t ar = a_row(r);
      ssrc = A.tiled ? A.scales + ar * 4 : A.scales + ar * KB;
      sstep = A.tiled ? A.rows * 4 : 4;
    } else {
      const int br = r - BM;
      const uint8_t* base = (NB == 2 && wave * 64 - BM >= BN) ? B.scales1 : B.scales0;
      const int n = min(n0 + (br % BN), N - 1);
      ssrc = base + (static_cast<int64_t>(tile.e) * nk * N + n) * 4;
      sstep = static_cast<int64_t>(N) * 4;
    }
  }
  // piece j < LPW of stage kt: 1 KB of codes; piece LPW: the 256-byte scale load
  auto issue_piece = [&](int kt, int j) {
    const uint32_t dst = smem_base + static_cast<uint32_t>((kt % STAGES) * STAGE_BYTES);
    if (j < LPW)
      dma16(src[j] + static_cast<int64_t>(kt) * kMxK, dst + (wave * LPW + j) * 1024);
    else
      dma4(ssrc + kt * sstep, dst + DATA + wave * 256);
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int j = 0; j < LPWT; ++j) issue_piece(kt, j);
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

  // Fragments and block scales of one 64-wide k step (s = 0, 1) of a stage:
  // the current ones and the next step's, read while the current MFMAs run.
  i32x8 ca[MI], cb[NB][NI], na[MI], nb[NB][NI];
  int cas[MI], cbs[NB][NI], nas[MI], nbs[NB][NI];
  auto frag = [&](i32x8& f, int& sv, const char* st, int s, int row) {
    const uint32_t* sc = reinterpret_cast<const uint32_t*>(st + DATA);
    const i32x4 lo = *reinterpret_cast<const i32x4*>(st + lds_chunk_byte<64>(row, 4 * s + hi));
    const i32x4 up = *reinterpret_cast<const i32x4*>(st + lds_chunk_byte<64>(row, 4 * s + 2 + hi));
    f = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
    sv = static_cast<int>(sc[row] >> (8 * (2 * s + hi)));
  };
  auto load_step = [&](i32x8 (&af)[MI], int (&as)[MI], i32x8 (&bf)[NB][NI], int (&bs)[NB][NI],
                       const char* st, int s) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) frag(af[mi], as[mi], st, s, wm * WTM + mi * 32 + l32);
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        frag(bf[q][ni], bs[q][ni], st, s, BM + q * BN + wn * WTN + ni * 32 + l32);
  };

  // Ring schedule (as in the bf16 GEMM): every slot holds a stage in flight
  // or being multiplied.  During the first 64-wide step of stage kt each
  // wave reads the rest of stage kt into registers; before the second step
  // the workgroup waits for stage kt+1 and passes one barrier, after which
  // stage kt's slot receives stage kt+STAGES while the second step's MFMAs
  // run: with SPREAD its pieces are spread evenly between those MFMAs,
  // else all are issued at the barrier.  The loop is split where the loads
  // stop, so that each iteration is one straight block (the fences around
  // the MFMAs only hold within a block, and the waits are constants).
  constexpr int MPK = NB * MI * NI;  // MFMAs per 64-wide step
  // MFMAs of the current fragments; with NEXT the next step's fragments are
  // read from (nst, ns) first; with LOADS stage `pend` is issued.
  auto step = [&](auto next_c, auto loads_c, const char* nst, int ns, int pend) {
    constexpr bool NEXT = decltype(next_c)::value, LOADS = decltype(loads_c)::value;
    if constexpr (LOADS && !SPREAD) issue(pend);
    if constexpr (NEXT) load_step(na, nas, nb, nbs, nst, ns);
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          mx_mfma(acc[q][mi][ni], cb[q][ni], ca[mi], cbs[q][ni], cas[mi]);
          if constexpr (LOADS && SPREAD) {
            const int pos = (q * MI + mi) * NI + ni;
#pragma unroll
            for (int j = 0; j < LPWT; ++j)
              if (j * MPK / LPWT == pos) issue_piece(pend, j);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
    if constexpr (NEXT) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        ca[mi] = na[mi];
        cas[mi] = nas[mi];
      }
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          cb[q][ni] = nb[q][ni];
          cbs[q][ni] = nbs[q][ni];
        }
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  auto slot = [&](int kt) { return smem + (kt % STAGES) * STAGE_BYTES; };

#pragma unroll
  for (int s = 0; s < STAGES; ++s)
    if (s < nk) issue(s);
  wait_stage<LPWT, STAGES>(min(STAGES - 1, nk - 1));
  block_barrier();
  load_step(ca, cas, cb, cbs, smem, 0);
  int kt = 0;
  for (; kt + STAGES < nk; ++kt) {  // a stage to load after each barrier
    step(T_{}, F_{}, slot(kt), 1, 0);
    wait_vmcnt<(STAGES - 2) * LPWT>();  // stage kt+1 has landed
    wait_lgkm0();
    block_barrier();                    // and every wave is done with stage kt
    step(T_{}, T_{}, slot(kt + 1), 0, kt + STAGES);
  }
  for (; kt + 1 < nk; ++kt) {  // nothing left to load
    step(T_{}, F_{}, slot(kt), 1, 0);
    wait_vmcnt<0>();
    wait_lgkm0();
    block_barrier();
    step(T_{}, F_{}, slot(kt + 1), 0, 0);
  }
  step(T_{}, F_{}, slot(nk - 1), 1, 0);  // last stage
  step(F_{}, F_{}, smem, 0, 0);
  // the accumulators are complete here: this keeps the last MFMAs (and
  // their fences) from being sunk into the epilogue's conditional stores
#pragma unroll
  for (int q = 0; q < NB; ++q)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) asm volatile("" : "+v"(acc[q][mi][ni]));

  mx_store<MI, NB, NI, WTM, WTN, FC1, CMB>(acc, tile, O, N, n0, wm, wn, l32, hi);
}

// Split-ring body of the queue launches (as the bf16 GEMM's gmm_tile_split):
// 128-row tiles with the activation rows in 2 LDS slots and the weight rows
// (256: BN of W_gate and of W_up, or BN = 256 of W_down) in 3, each slot
// holding its rows' 128 code bytes per stage and a padded block of scale
// dwords (one per lane of each loader's 4-byte load); the weight stream is
// issued two stages ahead, the activation rows one.  Waves 0-3 issue every
// direct load (per stage and loader: 4 activation pieces and one activation
// scale load, then 8 weight pieces and one weight scale load), waves 4-7 only
// multiply.  Sources are 32-bit offsets from SGPR bases (a loader's weight
// pieces step by 8 rows, so two offsets serve them).  Per stage kt: the
// first 64-wide step's MFMAs carry the weight group of stage kt+2; before the
// second step the loaders wait for stage kt+1 (that weight group may stay in
// flight), the workgroup passes one barrier, and the second step's MFMAs
// carry the activation group of stage kt+2.  Every scaled MFMA keeps its
// fence (mx_mfma).  The launcher checks that the offsets fit (a_rows * K and
// N * K below 2^31) and that N is a multiple of BN.
constexpr int kMxASlot = 128 * kMxK + 256 * 4;  // codes + 4 loaders x 64 scale dwords
constexpr int kMxBSlot = 256 * kMxK + 256 * 4;
constexpr int kMxSplitLds = 2 * kMxASlot + 3 * kMxBSlot;

template <int BN, int WM, int WN, bool FC1>
__device__ __forceinline__ void mx_tile_split(const Tile& tile, char* smem, const MxA& A,
                                              const MxB& B, const MxOut& O, int N, int K) {
  constexpr int BM = 128;
  constexpr int NB = FC1 ? 2 : 1;
  static_assert(NB * BN == 256, "256 weight rows per stage");
  static_assert(WM * WN == 8, "8 waves");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 32, NI = WTN / 32;
  constexpr int MPK = NB * MI * NI;  // MFMAs per 64-wide step
  static_assert(MPK == 4, "four MFMAs per step: the groups below are spread over them");
  constexpr int AG = 5, BG = 9;  // loads of a loader's activation / weight group
  const int n0 = tile.n0 * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, hi = lane >> 5;
  const uint32_t smem_base = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));
  const int nk = K / kMxK;
  const int64_t KB = K / 32;

  const bool loader = wave < 4;
  const int w = loader ? wave : 0;
  auto a_row = [&](int r) {
    int64_t ar = tile.row0 + min(r, tile.nrows - 1);
    if (A.gather) ar = min(max(static_cast<int64_t>(A.gather[ar]), int64_t(0)), A.rows - 1);
    return ar;
  };
  // codes: activation pieces 4w .. 4w+3 (rows 32w .. 32w+31), weight pieces
  // 8w .. 8w+7 (rows 64w .. 64w+63; FC1: w < 2 W_gate, w >= 2 W_up)
  const bool up = FC1 && w >= 2;
  const char* a_codes = uniform_ptr(A.codes);
  const char* b_codes =
      uniform_ptr((up ? B.codes1 : B.codes0) + static_cast<int64_t>(tile.e) * N * K);
  uint32_t aoff[4], boff[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int row, c;
    lds_piece<64>((4 * w + j) * 1024 + lane * 16, row, c);
    aoff[j] = static_cast<uint32_t>(a_row(row) * K + c * 16);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int row, c;
    lds_piece<64>((8 * w + j) * 1024 + lane * 16, row, c);
    boff[j] = static_cast<uint32_t>(static_cast<int64_t>(n0 + row % BN) * K + c * 16);
  }
  // scales: a loader's 4-byte load covers 64 rows (activation rows past 127
  // are the clamped last row, never read)
  const int64_t ar_s = a_row(min(64 * w + lane, BM - 1));
  const uint32_t asoff = static_cast<uint32_t>(A.tiled ? ar_s * 4 : ar_s * KB);
  const int64_t astep = A.tiled ? A.rows * 4 : 4;
  const char* a_scales = uniform_ptr(A.scales);
  const uint32_t bsoff = static_cast<uint32_t>((n0 + (64 * w + lane) % BN) * 4);
  const char* b_scales = uniform_ptr((up ? B.scales1 : B.scales0) +
                                     static_cast<int64_t>(tile.e) * nk * N * 4);
  auto slot_a = [&](int s) { return (s & 1) * kMxASlot; };
  auto slot_b = [&](int s) { return 2 * kMxASlot + (s % 3) * kMxBSlot; };
  // piece q of a group: activation q < 4 codes, q == 4 scales; weight q < 8
  // codes, q == 8 scales
  auto piece_a = [&](int s, int q) {
    const uint32_t dst = smem_base + slot_a(s);
    if (q < 4) dma16s(aoff[q], a_codes + static_cast<int64_t>(s) * kMxK, dst + (4 * w + q) * 1024);
    else dma4s(asoff, a_scales + s * astep, dst + BM * kMxK + w * 256);
  };
  auto piece_b = [&](int s, int q) {
    const uint32_t dst = smem_base + slot_b(s);
    if (q < 8)
      dma16s(boff[q & 1], b_codes + static_cast<int64_t>(s) * kMxK + static_cast<int64_t>(q & ~1) * 8 * K,
             dst + (8 * w + q) * 1024);
    else
      dma4s(bsoff, b_scales + static_cast<int64_t>(s) * N * 4, dst + 256 * kMxK + w * 256);
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
  i32x8 ca[MI], cb[NB][NI], na[MI], nb[NB][NI];
  int cas[MI], cbs[NB][NI], nas[MI], nbs[NB][NI];
  auto frag = [&](i32x8& f, int& sv, const char* st, int scale_at, int s, int row) {
    const uint32_t* sc = reinterpret_cast<const uint32_t*>(st + scale_at);
    const i32x4 lo = *reinterpret_cast<const i32x4*>(st + lds_chunk_byte<64>(row, 4 * s + hi));
    const i32x4 upr = *reinterpret_cast<const i32x4*>(st + lds_chunk_byte<64>(row, 4 * s + 2 + hi));
    f = __builtin_shufflevector(lo, upr, 0, 1, 2, 3, 4, 5, 6, 7);
    sv = static_cast<int>(sc[row] >> (8 * (2 * s + hi)));
  };
  auto load_step = [&](i32x8 (&af)[MI], int (&as)[MI], i32x8 (&bf)[NB][NI], int (&bs)[NB][NI],
                       int kt, int s) {
    const char* ast = smem + slot_a(kt);
    const char* bst = smem + slot_b(kt);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) frag(af[mi], as[mi], ast, BM * kMxK, s, wm * WTM + mi * 32 + l32);
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        frag(bf[q][ni], bs[q][ni], bst, 256 * kMxK, s, q * BN + wn * WTN + ni * 32 + l32);
  };

  // prologue: groups A0 B0 A1 B1 B2 (those that exist); then stage 0 must be in
  if (loader) {
#pragma unroll
    for (int q = 0; q < AG; ++q) piece_a(0, q);
#pragma unroll
    for (int q = 0; q < BG; ++q) piece_b(0, q);
    if (nk > 1) {
#pragma unroll
      for (int q = 0; q < AG; ++q) piece_a(1, q);
#pragma unroll
      for (int q = 0; q < BG; ++q) piece_b(1, q);
    }
    if (nk > 2) {
#pragma unroll
      for (int q = 0; q < BG; ++q) piece_b(2, q);
      wait_vmcnt<AG + 2 * BG>();
    } else if (nk > 1) {
      wait_vmcnt<AG + BG>();
    } else {
      wait_vmcnt<0>();
    }
  }
  block_barrier();
  load_step(ca, cas, cb, cbs, 0, 0);

  using T_ = std::true_type;
  using F_ = std::false_type;
  // one step's MFMAs of the current fragments, the next step's fragments read
  // first (NEXT: stage nkt, step ns); with IA (IB) the loader's activation
  // (weight) group of stage g goes out between the MFMAs (two or three loads
  // after each)
  auto step = [&](auto next_c, auto ia_c, auto ib_c, int nkt, int ns, int g) {
    constexpr bool NEXT = decltype(next_c)::value;
    constexpr bool IA = decltype(ia_c)::value, IB = decltype(ib_c)::value;
    if constexpr (NEXT) load_step(na, nas, nb, nbs, nkt, ns);
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          mx_mfma(acc[q][mi][ni], cb[q][ni], ca[mi], cbs[q][ni], cas[mi]);
          if constexpr (IA || IB) {
            constexpr int G = IA ? AG : BG;
            const int pos = (q * MI + mi) * NI + ni;
#pragma unroll
            for (int p = 0; p < G; ++p)
              if (p * MPK / G == pos) {
                if constexpr (IA) piece_a(g, p);
                else piece_b(g, p);
              }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
    if constexpr (NEXT) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        ca[mi] = na[mi];
        cas[mi] = nas[mi];
      }
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          cb[q][ni] = nb[q][ni];
          cbs[q][ni] = nbs[q][ni];
        }
    }
  };
  // Stage kt (LD: loader; IB0, IA1: the first / second step carries the
  // weight / activation group of stage kt+2; W: the wait leaves the weight
  // group of stage kt+2 in flight; LAST: no barrier).
  auto iter = [&](auto ld_c, auto ib0_c, auto ia1_c, auto w_c, auto last_c, int kt) {
    constexpr bool LD = decltype(ld_c)::value;
    constexpr bool IB0 = LD && decltype(ib0_c)::value, IA1 = LD && decltype(ia1_c)::value;
    constexpr bool W = decltype(w_c)::value, LAST = decltype(last_c)::value;
    step(T_{}, F_{}, std::integral_constant<bool, IB0>{}, kt, 1, kt + 2);
    if constexpr (!LAST) {
      if constexpr (LD) {
        if constexpr (W) wait_vmcnt<BG>();
        else wait_vmcnt<0>();
      }
      wait_lgkm0();
      block_barrier();
      step(T_{}, std::integral_constant<bool, IA1>{}, F_{}, kt + 1, 0, kt + 2);
    } else {
      step(F_{}, F_{}, F_{}, 0, 0, 0);
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
  // the accumulators are complete here: keep the last MFMAs (and their
  // fences) out of the epilogue's conditional stores
#pragma unroll
  for (int q = 0; q < NB; ++q)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) asm volatile("" : "+v"(acc[q][mi][ni]));
  mx_store<MI, NB, NI, WTM, WTN, FC1, false>(acc, tile, O, N, n0, wm, wn, l32, hi);
}


template <int BM_, int BN_, int WM, int WN, bool FC1, int STAGES, int SPREAD>
struct MxBody {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr bool combine = true;  // can run the top-1 combine epilogue
  static constexpr int lds = mx_lds_bytes<BM, BN, FC1, WM * WN, STAGES>();
  template <bool CMB>
  __device__ __forceinline__ static void run(const Tile& t, char* smem, const MxA& A, const MxB& B,
                                             const MxOut& O, int N, int K) {
    mx_tile<BM, BN, WM, WN, FC1, STAGES, SPREAD, CMB>(t, smem, A, B, O, N, K);
  }
};

// The queue launches' body: the split ring for tiles of more than 64 rows, a
// 64-row body (Small, the same weight columns) for the shorter ragged tiles,
// which then spend half the MFMA work on padding rows.
template <int BN_, int WM, int WN, bool FC1, class Small>
struct MxSplitBody {
  static_assert(Small::BN == BN_ && Small::BM == 64, "a 64-row body of the same columns");
  static constexpr int BM = 128, BN = BN_;
  static constexpr int lds = kMxSplitLds > Small::lds ? kMxSplitLds : Small::lds;
  static constexpr bool combine = false;  // no top-1 combine epilogue
  template <bool CMB>
  __device__ __forceinline__ static void run(const Tile& t, char* smem, const MxA& A, const MxB& B,
                                             const MxOut& O, int N, int K) {
    static_assert(!CMB, "queue launches only");
    if (t.nrows > 64) mx_tile_split<BN, WM, WN, FC1>(t, smem, A, B, O, N, K);
    else Small::template run<false>(t, smem, A, B, O, N, K);
  }
};

// The shared expert's dense GEMM (all tokens through one weight, [MC] §11)
// riding as the last tiles of a grouped launch, so that its tiles fill the
// tail of the routed experts' tiles: its operands, rows and sizes (tile
// order as dense_tile_at; A rows are not gathered).  With one workgroup per
// tile, the last `wgs` workgroups of the grid take these tiles.
struct MxDense {
  MxA A;
  MxB B;
  MxOut O;
  int64_t rows;
  int N, K;
  int wgs;
};

// Decode this workgroup's tile (Body::BM-row m-tiles, Body::BN columns), run the body.
// With the combine epilogue (CMB), the last zero_wgs workgroups write the
// dropped tokens' zero rows.  TAIL: the dense tail's tiles follow the routed
// ones.  QUEUE: one workgroup per CU takes tiles from the queue
// (queue_tiles) instead of one tile per workgroup.
template <bool FC1, class Body, bool CMB = false, bool TAIL = false, bool QUEUE = false>
__global__ void __launch_bounds__(512) gmm_mx_kernel(MxA A, MxB B, MxOut O,
                                                     const int32_t* __restrict__ counts, int E,
                                                     int N, int K, int64_t max_rows, int zero_wgs,
                                                     MxDense dn, int* __restrict__ queue) {
  static_assert(!(CMB && (TAIL || QUEUE)), "the combine epilogue runs in one-tile launches");
  if constexpr (CMB) {
    const int z = static_cast<int>(blockIdx.x) - static_cast<int>(gridDim.x - zero_wgs);
    if (z >= 0) {
      zero_dropped_rows(O.row_id_map, max_rows, O.cmb.out, O.cmb.T, N, z);
      return;
    }
  }
  constexpr int BM = Body::BM, BN = Body::BN;
  constexpr int DECODE_BYTES = (3 * kMaxExperts + 1) * 4 + 64;
  static_assert(Body::lds >= DECODE_BYTES, "decode scratch aliases the stages");
  __shared__ __attribute__((aligned(1024))) char smem[Body::lds];
  const int NT = (N + BN - 1) / BN;
  const int ntd = TAIL ? (dn.N + BN - 1) / BN : 0;
  // one call of the body per kernel; the operands are the routed experts'
  // or the dense tail's
  auto run = [&](Tile t, bool dense) {
    t.e = __builtin_amdgcn_readfirstlane(t.e);
    t.n0 = __builtin_amdgcn_readfirstlane(t.n0);
    t.nrows = __builtin_amdgcn_readfirstlane(t.nrows);
    t.row0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(t.row0)));
    MxA ta = A;
    MxB tb = B;
    MxOut to = O;
    int tn = N, tk = K;
    if (TAIL && dense) {
      ta = dn.A;
      tb = dn.B;
      to = dn.O;
      tn = dn.N;
      tk = dn.K;
    }
    Body::template run<CMB>(t, smem, ta, tb, to, tn, tk);
  };
  if constexpr (QUEUE) {
    __shared__ int p_toff[kPersistMaxExperts + 1], p_roff[kPersistMaxExperts],
        p_n[kPersistMaxExperts];
    __shared__ int s_kq;
    decode_to_tables<BM, 512>(counts, E, max_rows, smem, p_toff, p_roff, p_n);
    const int64_t routed = static_cast<int64_t>(p_toff[E]) * NT;
    const int64_t total = routed + (TAIL ? (dn.rows + BM - 1) / BM * ntd : 0);
    queue_tiles(queue, total, &s_kq, [&](int64_t L) {
      const bool dense = TAIL && L >= routed;
      run(dense ? dense_tile_at<BM, kDenseBand>(L - routed, ntd, dn.rows, 0)
                : tile_at<BM>(L, NT, E, p_toff, p_roff, p_n),
          dense);
    });
    return;
  }
  Tile tile;
  bool mine;
  // the tail starts at a multiple of 8, so d % 8 is this workgroup's XCD
  const int d = TAIL ? static_cast<int>(blockIdx.x) - static_cast<int>(gridDim.x - dn.wgs) : -1;
  if (TAIL && d >= 0) {
    const int64_t L = xcd_tile(d, (dn.rows + BM - 1) / BM * ntd);
    mine = L >= 0;
    if (mine) tile = dense_tile_at<BM, kDenseBand>(L, ntd, dn.rows, 0);
  } else {
    int* s_toff = reinterpret_cast<int*>(smem);
    int* s_roff = s_toff + kMaxExperts + 1;
    int* s_n = s_roff + kMaxExperts;
    int64_t* s_scan = reinterpret_cast<int64_t*>(s_n + kMaxExperts + 1);
    mine = decode_tile<BM, 512>(counts, E, max_rows, NT, s_toff, s_roff, s_n, s_scan, tile);
    __syncthreads();
  }
  // the decode is the same in every lane: say so to the compiler, so that
  // the tile loop runs as uniform (scalar) control flow
  if (!__builtin_amdgcn_readfirstlane(static_cast<int>(mine))) return;
  run(tile, TAIL && d >= 0);
}

// Bodies (8 waves, two per SIMD).  LDS per stage = rows * 128 + 2 KB of
// scales.  Loads are spread one per MFMA where a stage's loads fit into its
// two steps' MFMAs.  (256-row tiles need 128 accumulator registers per lane
// and, with the fp8 fragments, spill.)
using MxFc1B128 = MxBody<128, 128, 2, 4, true, 3, 1>;
using MxFc1B64 = MxBody<64, 128, 2, 4, true, 3, 0>;
using MxFc2B128w = MxBody<128, 256, 2, 4, false, 3, 1>;
using MxFc2B128 = MxBody<128, 128, 2, 4, false, 4, 0>;
using MxFc2B64w = MxBody<64, 256, 2, 4, false, 3, 0>;
// split-ring bodies of the queue launches
using MxFc1S = MxSplitBody<128, 2, 4, true, MxFc1B64>;
using MxFc2S = MxSplitBody<256, 2, 4, false, MxFc2B64w>;

// The split-ring queue bodies take 32-bit source offsets (codes of every
// activation row and of each expert's weight rows within 2^31 bytes of their
// base) and whole n-tiles (N a multiple of BN), for the routed experts and
// the dense tail alike.
bool mx_split_fits(const MxA& a, int64_t N, int64_t K, int BN, const MxDense* dense) {
  const int64_t lim = int64_t(1) << 31;
  if (a.rows * K > lim || N * K > lim || N % BN != 0 || a.rows * (K / 32) > lim) return false;
  if (dense && dense->rows > 0)
    return dense->rows * dense->K <= lim && int64_t(dense->N) * dense->K <= lim &&
           dense->N % BN == 0;
  return true;
}

// Queue launches from 192 rows per expert on average (as the bf16 GEMM).
bool use_queue_mx(int64_t max_rows, int64_t E) {
  return E > 1 && E <= kPersistMaxExperts && max_rows / E >= 192;
}

template <bool FC1, class Body>
void launch_mx(const MxA& a, const MxB& b, const MxOut& o, const int32_t* counts, int64_t E,
               int64_t N, int64_t K, int64_t max_rows, hipStream_t s,
               const MxDense* dense = nullptr, int* queue = nullptr) {
  const int64_t g = grid_for(max_rows, E, Body::BM, N, Body::BN);
  MxDense dn{MxA{}, MxB{}, MxOut{}, 0, 0, 0, 0};
  if (dense && dense->rows > 0) {
    dn = *dense;
    dn.wgs = static_cast<int>(grid_for(dn.rows, 1, Body::BM, dn.N, Body::BN));
  }
  const int e = static_cast<int>(E), n = static_cast<int>(N), k = static_cast<int>(K);
  if constexpr (!FC1 && Body::combine) {
    if (o.cmb.out) {  // callers pass neither a tail nor a queue
      const int64_t z = ceil_div(o.cmb.T, 8 * 16);  // 8 waves of 16 tokens
      hipLaunchKernelGGL((gmm_mx_kernel<FC1, Body, true>), dim3(static_cast<unsigned>(g + z)),
                         dim3(512), 0, s, a, b, o, counts, e, n, k, max_rows,
                         static_cast<int>(z), dn, static_cast<int*>(nullptr));
      return;
    }
  }
  if (queue && use_queue_mx(max_rows, E)) {
    if (g + dn.wgs == 0) return;
    const auto kern = dn.wgs > 0 ? gmm_mx_kernel<FC1, Body, false, true, true>
                                 : gmm_mx_kernel<FC1, Body, false, false, true>;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(persistent_grid(g + dn.wgs))), dim3(512), 0,
                       s, a, b, o, counts, e, n, k, max_rows, 0, dn, queue);
    return;
  }
  const auto kern = dn.wgs > 0 ? gmm_mx_kernel<FC1, Body, false, true>
                               : gmm_mx_kernel<FC1, Body>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(g + dn.wgs)), dim3(512), 0, s, a, b, o,
                     counts, e, n, k, max_rows, 0, dn, static_cast<int*>(nullptr));
}

moe_status validate_mx(const char* who, int64_t E, int64_t h, int64_t f, int64_t max_rows) {
  MOE_REQUIRE(E >= 1 && E <= kMaxExperts, MOE_ERR_ARG, "%s: E=%lld not in [1,%lld]", who,
              (long long)E, (long long)kMaxExperts);
  MOE_REQUIRE(max_rows >= 0 && max_rows < (int64_t(1) << 31), MOE_ERR_ARG, "%s: max_rows out of range",
              who);
  MOE_REQUIRE(h >= 128 && f >= 128 && h % 128 == 0 && f % 128 == 0, MOE_ERR_UNSUPPORTED,
              "%s: MXFP8 needs h and f to be multiples of 128 (h=%lld f=%lld)", who, (long long)h,
              (long long)f);
  MOE_REQUIRE(E * f < (int64_t(1) << 31) && E * h < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED,
              "%s: E*f or E*h too large", who);
  return MOE_OK;
}

void launch_fc2_mx(const MxA& a, const MxB& b, const MxOut& o, const int32_t* counts, int64_t E,
                   int64_t h, int64_t f, int64_t max_rows, hipStream_t s,
                   const MxDense* dense = nullptr, int* queue = nullptr) {
  const int64_t avg = max_rows / E;
  if (queue && !o.cmb.out && use_queue_mx(max_rows, E) && mx_split_fits(a, h, f, 256, dense))
    launch_mx<false, MxFc2S>(a, b, o, counts, E, h, f, max_rows, s, dense, queue);
  else if (avg >= 192)
    launch_mx<false, MxFc2B128w>(a, b, o, counts, E, h, f, max_rows, s, dense, queue);
  else if (avg >= 80)
    launch_mx<false, MxFc2B128>(a, b, o, counts, E, h, f, max_rows, s, dense, queue);
  else
    launch_mx<false, MxFc2B64w>(a, b, o, counts, E, h, f, max_rows, s, dense, queue);
}

void launch_fc1_mx(const MxA& a, const MxB& b, const MxOut& o, const int32_t* counts, int64_t E,
                   int64_t h, int64_t f, int64_t max_rows, hipStream_t s,
                   const MxDense* dense = nullptr, int* queue = nullptr) {
  if (queue && use_queue_mx(max_rows, E) && mx_split_fits(a, f, h, 128, dense))
    launch_mx<true, MxFc1S>(a, b, o, counts, E, f, h, max_rows, s, dense, queue);
  else if (max_rows / E >= 80)
    launch_mx<true, MxFc1B128>(a, b, o, counts, E, f, h, max_rows, s, dense, queue);
  else
    launch_mx<true, MxFc1B64>(a, b, o, counts, E, f, h, max_rows, s, dense, queue);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_grouped_fc1_swiglu_mxfp8(
    int64_t E, int64_t h, int64_t f, int64_t max_rows, int64_t T, const uint8_t* x_codes,
    const uint8_t* x_scales, const int32_t* sorted_token, const int32_t* tokens_per_expert,
    const uint8_t* wg_codes, const uint8_t* wg_scales, const uint8_t* wu_codes,
    const uint8_t* wu_scales, uint8_t* act_codes, uint8_t* act_scales, void* queue, void* stream) {
  moe_status st = validate_mx("moe_grouped_fc1_swiglu_mxfp8", E, h, f, max_rows);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(T >= 0 && T < (int64_t(1) << 31), MOE_ERR_ARG, "moe_grouped_fc1_swiglu_mxfp8: T out of range");
  if (max_rows == 0 || T == 0) return MOE_OK;
  MOE_REQUIRE(x_codes && x_scales && tokens_per_expert && wg_codes && wg_scales && wu_codes &&
                  wu_scales && act_codes && act_scales,
              MOE_ERR_ARG, "moe_grouped_fc1_swiglu_mxfp8: NULL tensor argument");
  const MxA a{x_codes, x_scales, sorted_token, sorted_token ? T : max_rows, false};
  const MxB b{wg_codes, wg_scales, wu_codes, wu_scales};
  const MxOut o{act_codes, act_scales, nullptr, max_rows};
  launch_fc1_mx(a, b, o, tokens_per_expert, E, h, f, max_rows, as_stream(stream), nullptr,
                static_cast<int*>(queue));
  return check_launch("moe_grouped_fc1_swiglu_mxfp8");
}

extern "C" moe_status moe_grouped_fc1_swiglu_mxfp8_shared(
    int64_t E, int64_t h, int64_t f, int64_t max_rows, int64_t T, const uint8_t* x_codes,
    const uint8_t* x_scales, const int32_t* sorted_token, const int32_t* tokens_per_expert,
    const uint8_t* wg_codes, const uint8_t* wg_scales, const uint8_t* wu_codes,
    const uint8_t* wu_scales, uint8_t* act_codes, uint8_t* act_scales, int64_t fs,
    const uint8_t* sg_codes, const uint8_t* sg_scales, const uint8_t* su_codes,
    const uint8_t* su_scales, uint8_t* shared_act_codes, uint8_t* shared_act_scales, void* queue,
    void* stream) {
  const char* who = "moe_grouped_fc1_swiglu_mxfp8_shared";
  moe_status st = validate_mx(who, E, h, f, max_rows);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(T >= 0 && T < (int64_t(1) << 31), MOE_ERR_ARG, "%s: T out of range", who);
  st = validate_mx(who, 1, h, fs, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(sorted_token, MOE_ERR_ARG, "%s: the routed rows are gathered (sorted_token)", who);
  MOE_REQUIRE(x_codes && x_scales && tokens_per_expert && wg_codes && wg_scales && wu_codes &&
                  wu_scales && sg_codes && sg_scales && su_codes && su_scales &&
                  shared_act_codes && shared_act_scales && (max_rows == 0 || (act_codes && act_scales)),
              MOE_ERR_ARG, "%s: NULL tensor argument", who);
  const MxA a{x_codes, x_scales, sorted_token, T, false};
  const MxB b{wg_codes, wg_scales, wu_codes, wu_scales};
  const MxOut o{act_codes, act_scales, nullptr, max_rows};
  const MxDense dn{MxA{x_codes, x_scales, nullptr, T, false},
                   MxB{sg_codes, sg_scales, su_codes, su_scales},
                   MxOut{shared_act_codes, shared_act_scales, nullptr, T},
                   T, static_cast<int>(fs), static_cast<int>(h), 0};
  launch_fc1_mx(a, b, o, tokens_per_expert, E, h, f, max_rows, as_stream(stream), &dn,
                static_cast<int*>(queue));
  return check_launch(who);
}

extern "C" moe_status moe_grouped_fc2_mxfp8(int64_t E, int64_t h, int64_t f, int64_t max_rows,
                                            const uint8_t* act_codes, const uint8_t* act_scales,
                                            const int32_t* tokens_per_expert, const uint8_t* wd_codes,
                                            const uint8_t* wd_scales, void* expert_out, void* queue,
                                            void* stream) {
  moe_status st = validate_mx("moe_grouped_fc2_mxfp8", E, h, f, max_rows);
  if (st != MOE_OK) return st;
  if (max_rows == 0) return MOE_OK;
  MOE_REQUIRE(act_codes && act_scales && tokens_per_expert && wd_codes && wd_scales && expert_out,
              MOE_ERR_ARG, "moe_grouped_fc2_mxfp8: NULL tensor argument");
  const MxA a{act_codes, act_scales, nullptr, max_rows, true};
  const MxB b{wd_codes, wd_scales, nullptr, nullptr};
  MxOut o{nullptr, nullptr, static_cast<uint16_t*>(expert_out), max_rows};
  launch_fc2_mx(a, b, o, tokens_per_expert, E, h, f, max_rows, as_stream(stream), nullptr,
                static_cast<int*>(queue));
  return check_launch("moe_grouped_fc2_mxfp8");
}

extern "C" moe_status moe_grouped_fc2_mxfp8_shared(
    int64_t E, int64_t h, int64_t f, int64_t max_rows, const uint8_t* act_codes,
    const uint8_t* act_scales, const int32_t* tokens_per_expert, const uint8_t* wd_codes,
    const uint8_t* wd_scales, void* expert_out, int64_t T, int64_t fs,
    const uint8_t* shared_act_codes, const uint8_t* shared_act_scales, const uint8_t* sd_codes,
    const uint8_t* sd_scales, void* shared_out, void* queue, void* stream) {
  const char* who = "moe_grouped_fc2_mxfp8_shared";
  moe_status st = validate_mx(who, E, h, f, max_rows);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(T >= 0 && T < (int64_t(1) << 31), MOE_ERR_ARG, "%s: T out of range", who);
  st = validate_mx(who, 1, h, fs, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(tokens_per_expert && wd_codes && wd_scales && shared_act_codes && shared_act_scales &&
                  sd_codes && sd_scales && shared_out &&
                  (max_rows == 0 || (act_codes && act_scales && expert_out)),
              MOE_ERR_ARG, "%s: NULL tensor argument", who);
  const MxA a{act_codes, act_scales, nullptr, max_rows, true};
  const MxB b{wd_codes, wd_scales, nullptr, nullptr};
  MxOut o{nullptr, nullptr, static_cast<uint16_t*>(expert_out), max_rows};
  const MxDense dn{MxA{shared_act_codes, shared_act_scales, nullptr, T, true},
                   MxB{sd_codes, sd_scales, nullptr, nullptr},
                   MxOut{nullptr, nullptr, static_cast<uint16_t*>(shared_out), T},
                   T, static_cast<int>(h), static_cast<int>(fs), 0};
  launch_fc2_mx(a, b, o, tokens_per_expert, E, h, f, max_rows, as_stream(stream), &dn,
                static_cast<int*>(queue));
  return check_launch(who);
}

extern "C" moe_status moe_grouped_fc2_combine_mxfp8(
    int64_t E, int64_t h, int64_t f, int64_t max_rows, int64_t T, const uint8_t* act_codes,
    const uint8_t* act_scales, const int32_t* tokens_per_expert, const uint8_t* wd_codes,
    const uint8_t* wd_scales, const float* permuted_probs, const int32_t* sorted_token,
    const int32_t* row_id_map, void* out, void* stream) {
  moe_status st = validate_mx("moe_grouped_fc2_combine_mxfp8", E, h, f, max_rows);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(T >= 0 && T < (int64_t(1) << 31), MOE_ERR_ARG,
              "moe_grouped_fc2_combine_mxfp8: T out of range");
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(tokens_per_expert && wd_codes && wd_scales && row_id_map && out, MOE_ERR_ARG,
              "moe_grouped_fc2_combine_mxfp8: NULL tensor argument");
  MOE_REQUIRE(max_rows == 0 || (act_codes && act_scales && permuted_probs && sorted_token),
              MOE_ERR_ARG, "moe_grouped_fc2_combine_mxfp8: NULL tensor argument");
  const MxA a{act_codes, act_scales, nullptr, max_rows, true};
  const MxB b{wd_codes, wd_scales, nullptr, nullptr};
  MxOut o{nullptr, nullptr, nullptr, max_rows};
  o.cmb = CombineEpi{sorted_token, permuted_probs, static_cast<uint16_t*>(out), T, row_id_map};
  o.row_id_map = row_id_map;
  launch_fc2_mx(a, b, o, tokens_per_expert, E, h, f, max_rows, as_stream(stream));
  return check_launch("moe_grouped_fc2_combine_mxfp8");
}
