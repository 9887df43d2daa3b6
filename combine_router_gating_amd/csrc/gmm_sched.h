// Device-side tile scheduler shared by the grouped GEMM kernels (bf16 and
// MXFP8): every workgroup scans tokens_per_expert in LDS and decodes its own
// tile (expert, n-tile, m-tile) from its workgroup id, with no host sync.
#pragma once

#include "moe_internal.h"

namespace moe {

constexpr int kGemmThreads = 256;

struct Tile {
  int e;       // expert
  int64_t row0;  // first global row of this m-tile
  int nrows;   // valid rows in this m-tile (>= 1)
  int n0;      // first output column
};

// Scan the per-expert row counts into LDS: s_roff[e] = first row of expert
// e, s_n[e] = its rows, s_toff[e] = its first m-tile (s_toff[E] = all m-tiles).
// Counts are clamped so that the rows stay within max_rows.  Returns the
// number of m-tiles; all threads of the workgroup call it.  The first wave
// does the work alone (64 experts per step, every count loaded up front,
// wave-level scans), so the workgroup passes a single barrier: this runs
// before every tile, on its critical path.
template <int BM, int NTHREADS = kGemmThreads>
__device__ int64_t decode_counts(const int32_t* __restrict__ counts, int E, int64_t max_rows,
                                 int* s_toff, int* s_roff, int* s_n, int64_t* scratch) {
  (void)scratch;
  constexpr int kSteps = kMaxExperts / 64;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int steps = (E + 63) / 64;
    int cv[kSteps];
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      const int e = j * 64 + lane;
      const int v = (j < steps && e < E) ? counts[e] : 0;
      cv[j] = v < 0 ? 0 : (v > max_rows ? static_cast<int>(max_rows) : v);
    }
    int64_t run = 0;  // rows before this step's experts
    int trun = 0;     // m-tiles before them
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      if (j >= steps) break;  // wave-uniform
      const int e = j * 64 + lane;
      int64_t incl = cv[j];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int64_t o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      const int64_t pre = run + incl - cv[j];
      run += __shfl(incl, 63, 64);
      const int64_t start = pre < max_rows ? pre : max_rows;
      const int64_t end = pre + cv[j] < max_rows ? pre + cv[j] : max_rows;
      const int n = static_cast<int>(end - start);
      const int tl = (n + BM - 1) / BM;
      int tincl = tl;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(tincl, off, 64);
        if (lane >= off) tincl += o;
      }
      if (e < E) {
        s_roff[e] = static_cast<int>(start);
        s_n[e] = n;
        s_toff[e] = trun + tincl - tl;
      }
      trun += __shfl(tincl, 63, 64);
    }
    if (lane == 0) s_toff[E] = trun;
  }
  __syncthreads();
  return s_toff[E];
}

// Logical tile L of the decoded counts; NT n-tiles per expert.  Order:
// expert -> n-tile -> m-tile, the m-tiles walked forward on even n-tiles and
// backward on odd ones, so that each tile shares an operand slab with the one
// before it (the weight slab within an n-tile, the activation rows across an
// n-tile change): a workgroup that takes the next tile from the queue starts
// a few microseconds after its predecessor, while the shared lines are still
// in L2.
template <int BM>
__device__ Tile tile_at(int64_t L, int NT, int E, const int* s_toff, const int* s_roff,
                        const int* s_n) {
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
  const int mi = static_cast<int>(r % mt);
  const int mtile = (nt & 1) ? mt - 1 - mi : mi;
  Tile tile;
  tile.e = e;
  tile.row0 = s_roff[e] + static_cast<int64_t>(mtile) * BM;
  tile.nrows = min(BM, s_n[e] - mtile * BM);
  tile.n0 = nt;
  return tile;
}

// The same decode by one wave with no LDS tables (for launches whose stages
// take all of LDS): lane l holds experts l, l + 64, l + 128 and l + 192
// (E <= kPersistMaxExperts), their clamped row counts scanned into row and
// m-tile offsets as decode_counts does.  WaveCounts::load runs on every lane
// of the wave; the results are wave-uniform.
struct WaveCounts {
  int n[4], roff[4], toff[4];
  int mtiles;  // all m-tiles (uniform)

  template <int BM>
  __device__ __forceinline__ void load(const int32_t* __restrict__ counts, int E, int64_t max_rows) {
    const int lane = threadIdx.x & 63;
    int cv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = j * 64 + lane;
      const int v = e < E ? counts[e] : 0;
      cv[j] = v < 0 ? 0 : (v > max_rows ? static_cast<int>(max_rows) : v);
    }
    int64_t run = 0;
    int trun = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t incl = cv[j];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int64_t o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      const int64_t pre = run + incl - cv[j];
      run += __shfl(incl, 63, 64);
      const int64_t start = pre < max_rows ? pre : max_rows;
      const int64_t end = pre + cv[j] < max_rows ? pre + cv[j] : max_rows;
      n[j] = static_cast<int>(end - start);
      roff[j] = static_cast<int>(start);
      const int tl = (n[j] + BM - 1) / BM;
      int tincl = tl;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(tincl, off, 64);
        if (lane >= off) tincl += o;
      }
      toff[j] = trun + tincl - tl;
      trun += __shfl(tincl, 63, 64);
    }
    mtiles = __builtin_amdgcn_readfirstlane(trun);
  }

  // Logical tile L < mtiles * NT, in tile_at's order.
  template <int BM>
  __device__ __forceinline__ Tile tile(int64_t L, int NT, int E) const {
    const int lane = threadIdx.x & 63;
    // e = (experts e' < E with toff[e'] * NT <= L) - 1: toff never decreases,
    // so this is the largest such e', which has tiles
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      cnt += __popcll(__ballot(j * 64 + lane < E && static_cast<int64_t>(toff[j]) * NT <= L));
    const int e = cnt - 1;
    const int j = e >> 6, l = e & 63;
    const auto pick = [&](const int (&v)[4]) {
      const int x = j == 0 ? v[0] : (j == 1 ? v[1] : (j == 2 ? v[2] : v[3]));
      return __builtin_amdgcn_readlane(x, l);
    };
    const int te = pick(toff), re = pick(roff), ne = pick(n);
    const int mt = (ne + BM - 1) / BM;
    const int64_t r = L - static_cast<int64_t>(te) * NT;
    const int nt = static_cast<int>(r / mt);
    const int mi = static_cast<int>(r % mt);
    const int mtile = (nt & 1) ? mt - 1 - mi : mi;
    Tile t;
    t.e = e;
    t.row0 = re + static_cast<int64_t>(mtile) * BM;
    t.nrows = min(BM, ne - mtile * BM);
    t.n0 = nt;
    return t;
  }
};

// Logical tiles are spread so that each XCD (workgroup id mod 8) runs a
// contiguous range of them (the weight slabs its CUs share stay in its L2):
// workgroup b's k-th tile (k = 0 for one tile per workgroup) is
// xcd_tile(b + k * grid, total).  Returns -1 when there is none.
__device__ __forceinline__ int64_t xcd_tile(int64_t bid, int64_t total) {
  const int64_t per = (total + 7) / 8;
  const int64_t slot = bid / 8;
  if (slot >= per) return -1;
  const int64_t L = (bid % 8) * per + slot;
  return L < total ? L : -1;
}

// Logical tile L of one dense GEMM (a single expert, e.g. the shared
// expert) in grouped order: m-tiles are taken in bands of G, and a band is
// walked n-tile by n-tile, so a run of consecutive tiles (one XCD's
// workgroups at a time) covers a G x (run / G) block of output tiles.  Its
// A and weight slabs are then a few each, not every m-tile of A against
// one weight slab (as the expert-major order gives with one expert).
template <int BM, int G>
__device__ Tile dense_tile_at(int64_t L, int NT, int64_t rows, int64_t row_base) {
  const int64_t MT = (rows + BM - 1) / BM;
  const int64_t band = L / (static_cast<int64_t>(G) * NT);
  const int64_t r = L - band * G * NT;
  const int64_t gm = min(static_cast<int64_t>(G), MT - band * G);  // m-tiles in this band
  const int64_t mt = band * G + r % gm;
  Tile tile;
  tile.e = 0;
  tile.row0 = row_base + mt * BM;
  tile.nrows = static_cast<int>(min(static_cast<int64_t>(BM), rows - mt * BM));
  tile.n0 = static_cast<int>(r / gm);
  return tile;
}

// Decode this workgroup's tile.  s_toff/s_roff/s_n: LDS arrays of E+1 / E+1 / E.
template <int BM, int NTHREADS = kGemmThreads>
__device__ bool decode_tile(const int32_t* __restrict__ counts, int E, int64_t max_rows, int NT,
                            int* s_toff, int* s_roff, int* s_n, int64_t* scratch, Tile& tile) {
  const int64_t total_tiles =
      decode_counts<BM, NTHREADS>(counts, E, max_rows, s_toff, s_roff, s_n, scratch);
  const int64_t L = xcd_tile(blockIdx.x, total_tiles * NT);
  if (L < 0) return false;
  tile = tile_at<BM>(L, NT, E, s_toff, s_roff, s_n);
  return true;
}

// Dense variant of decode_tile (E = 1): grouped order of dense_tile_at.
template <int BM, int G>
__device__ bool decode_dense_tile(const int32_t* __restrict__ counts, int64_t max_rows, int NT,
                                  int* s_n, Tile& tile) {
  if (threadIdx.x == 0) {
    const int v = counts[0];
    s_n[0] = v < 0 ? 0 : (v > max_rows ? static_cast<int>(max_rows) : v);
  }
  __syncthreads();
  const int64_t rows = s_n[0];
  const int64_t L = xcd_tile(blockIdx.x, (rows + BM - 1) / BM * NT);
  if (L < 0) return false;
  tile = dense_tile_at<BM, G>(L, NT, rows, 0);
  return true;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// FC2 with the K = 1 combine as its epilogue: row r of the tile goes to
// out[tok[r]] scaled by prob[r], rounded as the separate FC2 and combine
// round it (y to bf16 first, then p*y + 0 in fp32, then to bf16), so the
// result is bitwise theirs.  Only the row a token's combine slot names
// (rid[t] == r) is stored: with padding to capacity a token also owns rows
// of prob 0 in other experts, which the combine never reads and which
// must not overwrite its output.
struct CombineEpi {
  const int32_t* tok;
  const float* prob;
  uint16_t* out;
  int64_t T;
  const int32_t* rid;  // row_id_map [T] (K = 1)
  __device__ __forceinline__ int64_t token(int64_t r) const {
    return min(max(static_cast<int64_t>(tok[r]), int64_t(0)), T - 1);
  }
  // true when row r is its token's combine slot; *t receives the token
  __device__ __forceinline__ bool owns(int64_t r, int64_t* t) const {
    *t = token(r);
    return static_cast<int64_t>(rid[*t]) == r;
  }
};

__device__ __forceinline__ uint16_t combine_bf16(float p, float acc) {
  return f32_to_bf16_bits(fmaf(p, bf16_bits_to_f32(f32_to_bf16_bits(acc)), 0.f));
}

// Zero rows of the tokens with no kept row (row_id_map[t] outside
// [0, max_rows)); a wave covers 16 tokens (workgroup z: tokens from
// z * 16 * waves), 16-byte stores.
__device__ __forceinline__ void zero_dropped_rows(const int32_t* __restrict__ row_id_map,
                                                  int64_t max_rows, uint16_t* __restrict__ out,
                                                  int64_t T, int N, int z) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunks = N / 8;
  const int64_t t0 = (static_cast<int64_t>(z) * (blockDim.x >> 6) + wave) * 16;
  for (int i = 0; i < 16; ++i) {
    const int64_t t = t0 + i;
    if (t >= T) break;
    const int r = row_id_map[t];
    if (r >= 0 && r < max_rows) continue;
    uint4* row = reinterpret_cast<uint4*>(out + t * static_cast<int64_t>(N));
    for (int c = lane; c < chunks; c += 64) row[c] = make_uint4(0, 0, 0, 0);
  }
}

// m-tiles per band of the dense (single-expert) tile order
constexpr int kDenseBand = 8;
// experts whose decoded tables a persistent or queue launch keeps in LDS
constexpr int kPersistMaxExperts = 256;
// Tile queue (one workgroup per CU): the logical tiles are cut into groups
// of kQGroup consecutive tiles and XCD x owns groups x, x + 8, x + 16, ...;
// each XCD's counter sits kQStride ints (a 128-byte line) after the
// previous one, and the leave counter after the eight.
constexpr int kQGroup = 32;
constexpr int kQStride = 32;
// bf16 queue launches that carry the shared expert's dense tiles take them
// first: those tiles are all full and alike, and the launch then ends on
// the routed experts' tiles, whose ragged ones are shorter (measured on the
// DeepSeek-V3-shaped layer: FC1 -0.9 %, FC2 -1.6 %, the combine +5 %, as
// the shared expert's output is no longer the last thing FC2 wrote; the
// MXFP8 launches, where FC2 came out slower, keep the shared tiles last).
constexpr bool kDenseFirst = true;
static_assert(9 * kQStride * 4 <= MOE_GEMM_QUEUE_BYTES, "queue counters fit the buffer");

// Decode the counts once for a workgroup that runs many tiles: the scan
// uses `scratch` (LDS that the tile stages reuse afterwards), the tables it
// keeps are copied to p_toff [E+1], p_roff [E], p_n [E] (E <= kPersistMaxExperts).
template <int BM, int NTHREADS>
__device__ __forceinline__ void decode_to_tables(const int32_t* __restrict__ counts, int E,
                                                 int64_t max_rows, char* scratch, int* p_toff,
                                                 int* p_roff, int* p_n) {
  int* s_toff = reinterpret_cast<int*>(scratch);
  int* s_roff = s_toff + kMaxExperts + 1;
  int* s_n = s_roff + kMaxExperts;
  int64_t* s_scan = reinterpret_cast<int64_t*>(s_n + kMaxExperts + 1);
  decode_counts<BM, NTHREADS>(counts, E, max_rows, s_toff, s_roff, s_n, s_scan);
  for (int i = threadIdx.x; i <= E; i += blockDim.x) {
    p_toff[i] = s_toff[i];
    if (i < E) {
      p_roff[i] = s_roff[i];
      p_n[i] = s_n[i];
    }
  }
  __syncthreads();  // tables copied out of the scratch area
}

// A workgroup leaving the queue: the last of the launch to leave sets the
// counters back to zero, so the queue is zero again when the launch ends.
__device__ __forceinline__ void queue_leave(int* __restrict__ queue) {
  if (threadIdx.x == 0) {
    if (atomicAdd(queue + 8 * kQStride, 1) == static_cast<int>(gridDim.x) - 1) {
      for (int i = 0; i < 8; ++i) atomicExch(queue + i * kQStride, 0);
      atomicExch(queue + 8 * kQStride, 0);
    }
  }
}

// Runs run(L) for every logical tile L < total that this workgroup takes from
// the queue: its XCD's next tile while there is one, then the other XCDs'
// remaining tiles, one XCD after another (a counter only grows, so an XCD
// found empty stays empty), so that the XCDs end together.  Nothing waits
// on another workgroup; each leaves through queue_leave.  Uniform over the
// workgroup; s_kq is one int of LDS.
template <class Run>
__device__ __forceinline__ void queue_tiles(int* __restrict__ queue, int64_t total, int* s_kq,
                                            Run&& run) {
  const int x = static_cast<int>(blockIdx.x % 8);
  for (int v = 0; v < 8;) {
    const int xv = (x + v) % 8;
    if (threadIdx.x == 0) *s_kq = atomicAdd(queue + xv * kQStride, 1);
    __syncthreads();
    const int64_t kq = *s_kq;
    __syncthreads();  // s_kq is rewritten by the next take
    const int64_t L = ((kq / kQGroup) * 8 + xv) * kQGroup + kq % kQGroup;
    if (kq < 0 || L >= total) {  // uniform over the workgroup
      ++v;
      continue;
    }
    run(L);
    __syncthreads();  // every wave is past the tile before its stages are refilled
  }
  queue_leave(queue);
}

// Workgroups of a persistent or queue launch: one per CU (a multiple of 8,
// so that each workgroup stays on one XCD), never more than the tiles.
inline int64_t persistent_grid(int64_t tiles_grid) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 8)
    cus = 256;
  return tiles_grid < cus / 8 * 8 ? tiles_grid : cus / 8 * 8;
}

// Workgroups for the worst case: every expert's row count rounded up to BM
// (surplus workgroups exit after decoding), a multiple of 8 (one per XCD).
inline int64_t grid_for(int64_t max_rows, int64_t E, int BM, int64_t N, int BN) {
  const int64_t mtiles = (max_rows + E * (BM - 1)) / BM;
  const int64_t total = mtiles * ceil_div(N, BN);
  return ceil_div(total, 8) * 8;
}

}  // namespace moe
