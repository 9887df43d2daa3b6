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
// bf16 path: 256 threads (4 waves), tile BM x BN per weight matrix, k-steps
// of 64 staged through LDS (double-buffered, global loads for step k+1 in
// flight while step k is multiplied), v_mfma_f32_32x32x16_bf16 with fp32
// accumulation.  LDS rows are 128 bytes (8 chunks of 16 bytes) with chunk c
// of row r stored at c ^ (r & 7), so both the 16-byte writes and the
// 16-byte fragment reads are bank-conflict free.  The weight tile feeds the
// MFMA's first operand and the activation tile its second, so each lane
// ends with 4 consecutive output columns of one row (8-byte bf16 stores).
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Native 16-byte vector (HIP's uint4 is a struct, which defeats scalar
// replacement of register arrays).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BK = 64;

struct Tile {
  int e;       // expert
  int64_t row0;  // first global row of this m-tile
  int nrows;   // valid rows in this m-tile (>= 1)
  int n0;      // first output column
};

// Decode this workgroup's tile.  s_toff/s_roff/s_n: LDS arrays of E+1 / E+1 / E.
template <int BM>
__device__ bool decode_tile(const int32_t* __restrict__ counts, int E, int64_t max_rows, int NT,
                            int* s_toff, int* s_roff, int* s_n, int64_t* scratch, Tile& tile) {
  constexpr int PER = kMaxExperts / kThreads;  // experts per thread
  const int tid = threadIdx.x;
  int64_t c[PER];
  int64_t sum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = tid * PER + j;
    int64_t v = e < E ? static_cast<int64_t>(counts[e]) : 0;
    v = v < 0 ? 0 : (v > max_rows ? max_rows : v);
    c[j] = v;
    sum += v;
  }
  int64_t total_rows;
  int64_t pre = block_exclusive_scan256(sum, scratch, &total_rows);
  int tl[PER];
  int tsum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = tid * PER + j;
    const int64_t start = pre < max_rows ? pre : max_rows;
    const int64_t end = pre + c[j] < max_rows ? pre + c[j] : max_rows;
    const int n = static_cast<int>(end - start);
    tl[j] = (n + BM - 1) / BM;
    tsum += tl[j];
    if (e < E) {
      s_roff[e] = static_cast<int>(start);
      s_n[e] = n;
    }
    pre += c[j];
  }
  int64_t total_tiles;
  int tpre = static_cast<int>(block_exclusive_scan256(tsum, scratch, &total_tiles));
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = tid * PER + j;
    if (e < E) s_toff[e] = tpre;
    tpre += tl[j];
  }
  if (tid == 0) s_toff[E] = static_cast<int>(total_tiles);
  __syncthreads();

  const int64_t total = total_tiles * NT;
  const int64_t per = (total + 7) / 8;
  const int64_t bid = blockIdx.x;
  const int64_t slot = bid / 8;
  if (slot >= per) return false;
  const int64_t L = (bid % 8) * per + slot;
  if (L >= total) return false;
  // largest e with s_toff[e] * NT <= L (experts without tiles are skipped)
  int lo = 0, hi = E;  // invariant: s_toff[lo]*NT <= L < s_toff[hi]*NT
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (static_cast<int64_t>(s_toff[mid]) * NT <= L) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int mt = s_toff[e + 1] - s_toff[e];
  const int64_t r = L - static_cast<int64_t>(s_toff[e]) * NT;
  const int nt = static_cast<int>(r / mt);
  const int mtile = static_cast<int>(r % mt);
  tile.e = e;
  tile.row0 = s_roff[e] + static_cast<int64_t>(mtile) * BM;
  tile.nrows = min(BM, s_n[e] - mtile * BM);
  tile.n0 = nt;
  return true;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Global -> registers for one k-step: A rows, then the weight rows (the
// first BN from B0, the next BN from B1 when the tile holds two matrices).
template <int A_LD, int B_LD, int BN>
__device__ __forceinline__ void gmm_gload(u32x4 (&ra)[A_LD], u32x4 (&rb)[B_LD],
                                          const uint16_t* a_base, const uint16_t* b0_base,
                                          const uint16_t* b1_base, const uint32_t (&a_off)[A_LD],
                                          const uint32_t (&b_off)[B_LD], int kt) {
  const uint32_t ko = static_cast<uint32_t>(kt) * BK;
#pragma unroll
  for (int i = 0; i < A_LD; ++i) ra[i] = *reinterpret_cast<const u32x4*>(a_base + a_off[i] + ko);
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const uint16_t* bb = ((32 * i) / BN == 0) ? b0_base : b1_base;
    rb[i] = *reinterpret_cast<const u32x4*>(bb + b_off[i] + ko);
  }
}

// Registers -> one LDS stage, chunk c of row r at c ^ (r & 7).
template <int A_LD, int B_LD, int BM>
__device__ __forceinline__ void gmm_sstore(u32x4* sdst, const u32x4 (&ra)[A_LD],
                                           const u32x4 (&rb)[B_LD], int r, int c) {
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int lr = r + 32 * i;
    sdst[lr * 8 + (c ^ (lr & 7))] = ra[i];
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int br = BM + r + 32 * i;
    sdst[br * 8 + (c ^ (br & 7))] = rb[i];
  }
}

// ----------------------------------------------------------------- bf16 MFMA
template <int BM, int BN, int WM, int WN, bool FC1>
__global__ void __launch_bounds__(kThreads) gmm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1,
    uint16_t* __restrict__ C, const int32_t* __restrict__ counts, int E, int N, int K,
    int64_t max_rows) {
  constexpr int NB = FC1 ? 2 : 1;
  constexpr int BROWS = NB * BN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 32, NI = WTN / 32;
  constexpr int A_LD = BM / 32, B_LD = BROWS / 32;
  constexpr int STAGE = (BM + BROWS) * 8;  // 16-byte chunks per stage
  static_assert(WM * WN == 4, "4 waves");
  static_assert(MI >= 1 && NI >= 1, "wave tile must be at least 32x32");

  __shared__ u32x4 smem[2 * STAGE];
  __shared__ int s_toff[kMaxExperts + 1];
  __shared__ int s_roff[kMaxExperts];
  __shared__ int s_n[kMaxExperts];
  __shared__ int64_t s_scan[8];

  const int NT = (N + BN - 1) / BN;
  Tile tile;
  if (!decode_tile<BM>(counts, E, max_rows, NT, s_toff, s_roff, s_n, s_scan, tile)) return;
  const int n0 = tile.n0 * BN;

  const int tid = threadIdx.x;
  const int c = tid & 7, r = tid >> 3;  // chunk within a 128-byte row; row 0..31
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // Global sources: wave-uniform bases plus 32-bit per-thread offsets.  Rows
  // past the tile's valid rows (or past N) are clamped in range: they are
  // computed but never stored.
  const uint16_t* a_base = A + tile.row0 * static_cast<int64_t>(K);
  const int64_t b_expert = static_cast<int64_t>(tile.e) * N * K;
  const uint16_t* b0_base = B0 + b_expert;
  const uint16_t* b1_base = (NB == 2 ? B1 : B0) + b_expert;
  uint32_t a_off[A_LD], b_off[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int lr = min(r + 32 * i, tile.nrows - 1);
    a_off[i] = static_cast<uint32_t>(lr) * K + c * 8;
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int br = (r + 32 * i) % BN;  // row within one weight matrix
    const int n = min(n0 + br, N - 1);
    b_off[i] = static_cast<uint32_t>(n) * K + c * 8;
  }

  f32x16 acc[NB][MI][NI];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[b][mi][ni][q] = 0.f;

  u32x4 ra[A_LD], rb[B_LD];

  const int nk = K / BK;
  gmm_gload<A_LD, B_LD, BN>(ra, rb, a_base, b0_base, b1_base, a_off, b_off, 0);
  gmm_sstore<A_LD, B_LD, BM>(smem, ra, rb, r, c);
  __syncthreads();
  const int lr32 = lane & 31, hi = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gmm_gload<A_LD, B_LD, BN>(ra, rb, a_base, b0_base, b1_base, a_off, b_off, kt + 1);
    const u32x4* s = smem + (kt & 1) * STAGE;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ch = kk * 2 + hi;
      bf16x8 af[MI], bfr[NB][NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = wm * WTM + mi * 32 + lr32;
        const u32x4 v = s[row * 8 + (ch ^ (row & 7))];
        af[mi] = *reinterpret_cast<const bf16x8*>(&v);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int row = BM + b * BN + wn * WTN + ni * 32 + lr32;
          const u32x4 v = s[row * 8 + (ch ^ (row & 7))];
          bfr[b][ni] = *reinterpret_cast<const bf16x8*>(&v);
        }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[b][mi][ni] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[b][ni], af[mi], acc[b][mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) gmm_sstore<A_LD, B_LD, BM>(smem + ((kt + 1) & 1) * STAGE, ra, rb, r, c);
    __syncthreads();
  }

  // epilogue: lane holds C[m = lr32][n = 8*g + 4*hi + q] of each 32x32 block
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int ml = wm * WTM + mi * 32 + lr32;
    if (ml >= tile.nrows) continue;
    uint16_t* crow = C + (tile.row0 + ml) * static_cast<int64_t>(N);
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

// ----------------------------------------------------------------- fp32 SIMT
// For fp32 layers: 64x64 tiles, 16x16 threads with 4x4 outputs each (per
// weight matrix), k-slabs of 16 through LDS; any N and K.
constexpr int FM = 64, FN = 64, FK = 16;

template <bool FC1>
__global__ void __launch_bounds__(kThreads) gmm_f32_kernel(const float* __restrict__ A,
                                                           const float* __restrict__ B0,
                                                           const float* __restrict__ B1,
                                                           float* __restrict__ C,
                                                           const int32_t* __restrict__ counts,
                                                           int E, int N, int K, int64_t max_rows) {
  constexpr int NB = FC1 ? 2 : 1;
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
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  float acc[NB][4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FK) {
    for (int i = tid; i < FM * FK; i += kThreads) {
      const int rr = i / FK, kk = i % FK;
      const int k = k0 + kk;
      const int lr = min(rr, tile.nrows - 1);
      as[kk][rr] = k < K ? A[(tile.row0 + lr) * static_cast<int64_t>(K) + k] : 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float* B = b == 0 ? B0 : B1;
        const int n = min(n0 + rr, N - 1);
        bs[b][kk][rr] = k < K ? B[(static_cast<int64_t>(tile.e) * N + n) * K + k] : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; ++kk) {
      float av[4], bv[NB][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = as[kk][ty * 4 + i];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[b][j] = bs[b][kk][tx * 4 + j];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[b][i][j] = fmaf(av[i], bv[b][j], acc[b][i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ml = ty * 4 + i;
    if (ml >= tile.nrows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      const float v = FC1 ? silu_mul(acc[0][i][j], acc[NB - 1][i][j]) : acc[0][i][j];
      C[(tile.row0 + ml) * static_cast<int64_t>(N) + n] = v;
    }
  }
}

// ----------------------------------------------------------------- launch
int64_t grid_for(int64_t max_rows, int64_t E, int BM, int64_t N, int BN) {
  const int64_t mtiles = (max_rows + E * (BM - 1)) / BM;
  const int64_t total = mtiles * ceil_div(N, BN);
  return ceil_div(total, 8) * 8;
}

template <int BM, int BN, int WM, int WN, bool FC1>
void launch_bf16(const void* A, const void* B0, const void* B1, void* C, const int32_t* counts,
                 int64_t E, int64_t N, int64_t K, int64_t max_rows, hipStream_t s) {
  const int64_t g = grid_for(max_rows, E, BM, N, BN);
  hipLaunchKernelGGL((gmm_bf16_kernel<BM, BN, WM, WN, FC1>), dim3(static_cast<unsigned>(g)),
                     dim3(kThreads), 0, s, static_cast<const uint16_t*>(A),
                     static_cast<const uint16_t*>(B0), static_cast<const uint16_t*>(B1),
                     static_cast<uint16_t*>(C), counts, static_cast<int>(E), static_cast<int>(N),
                     static_cast<int>(K), max_rows);
}

template <bool FC1>
void launch_f32(const void* A, const void* B0, const void* B1, void* C, const int32_t* counts,
                int64_t E, int64_t N, int64_t K, int64_t max_rows, hipStream_t s) {
  const int64_t g = grid_for(max_rows, E, FM, N, FN);
  hipLaunchKernelGGL((gmm_f32_kernel<FC1>), dim3(static_cast<unsigned>(g)), dim3(kThreads), 0, s,
                     static_cast<const float*>(A), static_cast<const float*>(B0),
                     static_cast<const float*>(B1), static_cast<float*>(C), counts,
                     static_cast<int>(E), static_cast<int>(N), static_cast<int>(K), max_rows);
}

// Tile height from the average rows per expert (known on the host without
// reading the device counts): tall tiles amortise weight reads when experts
// are large; short tiles waste fewer MFMA cycles on padding when they are not.
int pick_bm(int64_t max_rows, int64_t E) {
  const int64_t avg = max_rows / E;
  if (avg >= 512) return 256;
  if (avg >= 192) return 128;
  return 64;
}

template <bool FC1>
void launch_gemm(int32_t dtype, const void* A, const void* B0, const void* B1, void* C,
                 const int32_t* counts, int64_t E, int64_t N, int64_t K, int64_t max_rows,
                 hipStream_t s) {
  if (dtype == MOE_F32) {
    launch_f32<FC1>(A, B0, B1, C, counts, E, N, K, max_rows, s);
    return;
  }
  const int bm = pick_bm(max_rows, E);
  if constexpr (FC1) {
    if (bm == 256) launch_bf16<256, 128, 2, 2, FC1>(A, B0, B1, C, counts, E, N, K, max_rows, s);
    else if (bm == 128) launch_bf16<128, 128, 2, 2, FC1>(A, B0, B1, C, counts, E, N, K, max_rows, s);
    else launch_bf16<64, 128, 1, 4, FC1>(A, B0, B1, C, counts, E, N, K, max_rows, s);
  } else {
    if (bm == 256) launch_bf16<256, 256, 2, 2, FC1>(A, B0, B1, C, counts, E, N, K, max_rows, s);
    else if (bm == 128) launch_bf16<128, 256, 2, 2, FC1>(A, B0, B1, C, counts, E, N, K, max_rows, s);
    else launch_bf16<64, 256, 1, 4, FC1>(A, B0, B1, C, counts, E, N, K, max_rows, s);
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
                                             const void* w_up, void* act, void* stream) {
  moe_status st = validate("moe_grouped_fc1_swiglu", E, h, f, max_rows, dtype);
  if (st != MOE_OK) return st;
  if (max_rows == 0) return MOE_OK;
  MOE_REQUIRE(permuted_x && tokens_per_expert && w_gate && w_up && act, MOE_ERR_ARG,
              "moe_grouped_fc1_swiglu: NULL tensor argument");
  launch_gemm<true>(dtype, permuted_x, w_gate, w_up, act, tokens_per_expert, E, f, h, max_rows,
                    as_stream(stream));
  return check_launch("moe_grouped_fc1_swiglu");
}

extern "C" moe_status moe_grouped_fc2(int64_t E, int64_t h, int64_t f, int64_t max_rows,
                                      int32_t dtype, const void* act,
                                      const int32_t* tokens_per_expert, const void* w_down,
                                      void* expert_out, void* stream) {
  moe_status st = validate("moe_grouped_fc2", E, h, f, max_rows, dtype);
  if (st != MOE_OK) return st;
  if (max_rows == 0) return MOE_OK;
  MOE_REQUIRE(act && tokens_per_expert && w_down && expert_out, MOE_ERR_ARG,
              "moe_grouped_fc2: NULL tensor argument");
  launch_gemm<false>(dtype, act, w_down, nullptr, expert_out, tokens_per_expert, E, h, f, max_rows,
                     as_stream(stream));
  return check_launch("moe_grouped_fc2");
}

extern "C" moe_status moe_grouped_mlp(int64_t E, int64_t h, int64_t f, int64_t max_rows,
                                      int32_t dtype, const void* permuted_x,
                                      const int32_t* tokens_per_expert, const void* w_gate,
                                      const void* w_up, const void* w_down, void* act,
                                      void* expert_out, void* stream) {
  moe_status st = moe_grouped_fc1_swiglu(E, h, f, max_rows, dtype, permuted_x, tokens_per_expert,
                                         w_gate, w_up, act, stream);
  if (st != MOE_OK) return st;
  return moe_grouped_fc2(E, h, f, max_rows, dtype, act, tokens_per_expert, w_down, expert_out,
                         stream);
}
