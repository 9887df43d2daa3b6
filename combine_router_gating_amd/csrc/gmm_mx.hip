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
// bytes, all filled by direct global->LDS loads.
#include "gmm_sched.h"
#include "mx_codec.h"

namespace moe {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMxK = 128;  // k per stage: 128 E4M3 bytes per row, 4 scale bytes

// Direct 4-byte global -> LDS load: lane i writes LDS bytes [base + 4 i, +4).
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
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
};

template <int BM, int BN, bool FC1, int NW, int STAGES>
constexpr int mx_lds_bytes() {
  return STAGES * ((BM + (FC1 ? 2 : 1) * BN) * kMxK + NW * 64 * 4);
}

// One output tile (BM rows of one expert x BN columns).
template <int BM, int BN, int WM, int WN, bool FC1, int STAGES>
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
  const int64_t b_expert = static_cast<int64_t>(tile.e) * N;

  // source row (clamped in range; padding rows are computed, never stored)
  auto a_row = [&](int r) {
    int64_t ar = tile.row0 + min(r, tile.nrows - 1);
    if (A.gather) ar = min(max(static_cast<int64_t>(A.gather[ar]), int64_t(0)), A.rows - 1);
    return ar;
  };
  const uint8_t* src[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    int row, c;
    lds_piece<64>((wave * LPW + j) * 1024 + lane * 16, row, c);
    if (row < BM) {
      src[j] = A.codes + a_row(row) * K + c * 16;
    } else {
      const int br = row - BM;
      const uint8_t* base = (NB == 2 && br >= BN) ? B.codes1 : B.codes0;
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
    if (r < BM) {
      const int64_t ar = a_row(r);
      ssrc = A.tiled ? A.scales + ar * 4 : A.scales + ar * KB;
      sstep = A.tiled ? A.rows * 4 : 4;
    } else {
      const int br = r - BM;
      const uint8_t* base = (NB == 2 && br >= BN) ? B.scales1 : B.scales0;
      const int n = min(n0 + (br % BN), N - 1);
      ssrc = base + (static_cast<int64_t>(tile.e) * (K / kMxK) * N + n) * 4;
      sstep = static_cast<int64_t>(N) * 4;
    }
  }
  auto issue = [&](int kt) {
    const uint32_t dst = smem_base + static_cast<uint32_t>((kt % STAGES) * STAGE_BYTES);
    const int64_t ko = static_cast<int64_t>(kt) * kMxK;
#pragma unroll
    for (int j = 0; j < LPW; ++j) dma16(src[j] + ko, dst + (wave * LPW + j) * 1024);
    dma4(ssrc + kt * sstep, dst + DATA + wave * 256);
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

  const int nk = K / kMxK;
#pragma unroll
  for (int s = 0; s < STAGES; ++s)
    if (s < nk) issue(s);
  for (int kt = 0; kt < nk; ++kt) {
    wait_stage<LPWT, STAGES>(min(kt + STAGES - 1, nk - 1) - kt);
    block_barrier();
    const char* st = smem + (kt % STAGES) * STAGE_BYTES;
    const uint32_t* sc = reinterpret_cast<const uint32_t*>(st + DATA);
#pragma unroll
    for (int s = 0; s < kMxK / 64; ++s) {
      i32x8 af[MI], bf[NB][NI];
      int as[MI], bs[NB][NI];
      const int shift = 8 * (2 * s + hi);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = wm * WTM + mi * 32 + l32;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(st + lds_chunk_byte<64>(row, 4 * s + hi));
        const i32x4 up = *reinterpret_cast<const i32x4*>(st + lds_chunk_byte<64>(row, 4 * s + 2 + hi));
        af[mi] = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
        as[mi] = static_cast<int>(sc[row] >> shift);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int row = BM + nb * BN + wn * WTN + ni * 32 + l32;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(st + lds_chunk_byte<64>(row, 4 * s + hi));
          const i32x4 up =
              *reinterpret_cast<const i32x4*>(st + lds_chunk_byte<64>(row, 4 * s + 2 + hi));
          bf[nb][ni] = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
          bs[nb][ni] = static_cast<int>(sc[row] >> shift);
        }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[nb][mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bf[nb][ni], af[mi], acc[nb][mi][ni], 0, 0, 0, bs[nb][ni], 0, as[mi]);
    }
    if (kt + STAGES < nk) {
      wait_lgkm0();
      block_barrier();  // every wave is done with this slot
      issue(kt + STAGES);
    }
  }

  // epilogue: lane holds C[m = l32][n = 8g + 4*hi + q] of each 32x32 block
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

template <int BM, int BN, int WM, int WN, bool FC1, int STAGES>
struct MxBody {
  static constexpr int lds = mx_lds_bytes<BM, BN, FC1, WM * WN, STAGES>();
  __device__ __forceinline__ static void run(const Tile& t, char* smem, const MxA& A, const MxB& B,
                                             const MxOut& O, int N, int K) {
    mx_tile<BM, BN, WM, WN, FC1, STAGES>(t, smem, A, B, O, N, K);
  }
};

// Decode the tile with BMAX-row m-tiles, then run a body (ragged tails of
// 256-row launches run the 128- or 64-row body).
template <bool FC1, int BMAX, int BN, class Body256, class Body128, class Body64>
__global__ void __launch_bounds__(512) gmm_mx_kernel(MxA A, MxB B, MxOut O,
                                                     const int32_t* __restrict__ counts, int E,
                                                     int N, int K, int64_t max_rows) {
  constexpr int L256 = Body256::lds > Body128::lds ? Body256::lds : Body128::lds;
  constexpr int LDS = BMAX == 256 ? (L256 > Body64::lds ? L256 : Body64::lds)
                                 : (BMAX == 128 ? Body128::lds : Body64::lds);
  constexpr int DECODE_BYTES = (3 * kMaxExperts + 1) * 4 + 64;
  static_assert(LDS >= DECODE_BYTES, "decode scratch aliases the stages");
  __shared__ __attribute__((aligned(1024))) char smem[LDS];
  const int NT = (N + BN - 1) / BN;
  Tile tile;
  {
    int* s_toff = reinterpret_cast<int*>(smem);
    int* s_roff = s_toff + kMaxExperts + 1;
    int* s_n = s_roff + kMaxExperts;
    int64_t* s_scan = reinterpret_cast<int64_t*>(s_n + kMaxExperts + 1);
    const bool mine = decode_tile<BMAX, 512>(counts, E, max_rows, NT, s_toff, s_roff, s_n, s_scan, tile);
    __syncthreads();
    if (!mine) return;
  }
  tile.nrows = __builtin_amdgcn_readfirstlane(tile.nrows);
  if constexpr (BMAX == 256) {
    if (tile.nrows > 128) Body256::run(tile, smem, A, B, O, N, K);
    else if (tile.nrows > 64) Body128::run(tile, smem, A, B, O, N, K);
    else Body64::run(tile, smem, A, B, O, N, K);
  } else if constexpr (BMAX == 128) {
    Body128::run(tile, smem, A, B, O, N, K);
  } else {
    Body64::run(tile, smem, A, B, O, N, K);
  }
}

// Bodies (8 waves).  LDS per stage = rows * 128 + 2 KB of scales.
using MxFc1B256 = MxBody<256, 128, 2, 4, true, 2>;
using MxFc1B128 = MxBody<128, 128, 2, 4, true, 3>;
using MxFc1B64 = MxBody<64, 128, 2, 4, true, 3>;
using MxFc2B256 = MxBody<256, 256, 4, 2, false, 2>;
using MxFc2B128w = MxBody<128, 256, 2, 4, false, 3>;
using MxFc2B64w = MxBody<64, 256, 2, 4, false, 3>;
using MxFc2B128 = MxBody<128, 128, 2, 4, false, 4>;

template <bool FC1, int BMAX, int BN, class B256, class B128, class B64>
void launch_mx(const MxA& a, const MxB& b, const MxOut& o, const int32_t* counts, int64_t E,
               int64_t N, int64_t K, int64_t max_rows, hipStream_t s) {
  const int64_t g = grid_for(max_rows, E, BMAX, N, BN);
  hipLaunchKernelGGL((gmm_mx_kernel<FC1, BMAX, BN, B256, B128, B64>), dim3(static_cast<unsigned>(g)),
                     dim3(512), 0, s, a, b, o, counts, static_cast<int>(E), static_cast<int>(N),
                     static_cast<int>(K), max_rows);
}

int pick_bm_mx(int64_t max_rows, int64_t E) {
  const int64_t avg = max_rows / E;
  if (avg >= 192) return 256;
  if (avg >= 80) return 128;
  return 64;
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

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_grouped_fc1_swiglu_mxfp8(
    int64_t E, int64_t h, int64_t f, int64_t max_rows, int64_t T, const uint8_t* x_codes,
    const uint8_t* x_scales, const int32_t* sorted_token, const int32_t* tokens_per_expert,
    const uint8_t* wg_codes, const uint8_t* wg_scales, const uint8_t* wu_codes,
    const uint8_t* wu_scales, uint8_t* act_codes, uint8_t* act_scales, void* stream) {
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
  const hipStream_t s = as_stream(stream);
  const int bm = pick_bm_mx(max_rows, E);
  if (bm == 256)
    launch_mx<true, 256, 128, MxFc1B256, MxFc1B128, MxFc1B64>(a, b, o, tokens_per_expert, E, f, h, max_rows, s);
  else if (bm == 128)
    launch_mx<true, 128, 128, MxFc1B128, MxFc1B128, MxFc1B128>(a, b, o, tokens_per_expert, E, f, h, max_rows, s);
  else
    launch_mx<true, 64, 128, MxFc1B64, MxFc1B64, MxFc1B64>(a, b, o, tokens_per_expert, E, f, h, max_rows, s);
  return check_launch("moe_grouped_fc1_swiglu_mxfp8");
}

extern "C" moe_status moe_grouped_fc2_mxfp8(int64_t E, int64_t h, int64_t f, int64_t max_rows,
                                            const uint8_t* act_codes, const uint8_t* act_scales,
                                            const int32_t* tokens_per_expert, const uint8_t* wd_codes,
                                            const uint8_t* wd_scales, void* expert_out,
                                            void* stream) {
  moe_status st = validate_mx("moe_grouped_fc2_mxfp8", E, h, f, max_rows);
  if (st != MOE_OK) return st;
  if (max_rows == 0) return MOE_OK;
  MOE_REQUIRE(act_codes && act_scales && tokens_per_expert && wd_codes && wd_scales && expert_out,
              MOE_ERR_ARG, "moe_grouped_fc2_mxfp8: NULL tensor argument");
  const MxA a{act_codes, act_scales, nullptr, max_rows, true};
  const MxB b{wd_codes, wd_scales, nullptr, nullptr};
  const MxOut o{nullptr, nullptr, static_cast<uint16_t*>(expert_out), max_rows};
  const hipStream_t s = as_stream(stream);
  const int bm = pick_bm_mx(max_rows, E);
  if (bm == 256)
    launch_mx<false, 256, 256, MxFc2B256, MxFc2B128w, MxFc2B64w>(a, b, o, tokens_per_expert, E, h, f, max_rows, s);
  else if (bm == 128)
    launch_mx<false, 128, 128, MxFc2B128, MxFc2B128, MxFc2B128>(a, b, o, tokens_per_expert, E, h, f, max_rows, s);
  else
    launch_mx<false, 64, 256, MxFc2B64w, MxFc2B64w, MxFc2B64w>(a, b, o, tokens_per_expert, E, h, f, max_rows, s);
  return check_launch("moe_grouped_fc2_mxfp8");
}
