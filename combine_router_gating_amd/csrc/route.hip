// Router forward: fp32 gating linear, score function, top-k, capacity drop.
//
// Megatron Core MoE 源码路径解析 §3: the router casts its input to fp32 and
// applies a linear gate (optional bias) to get [T,E] logits.  §4/§5: top-k
// routing with a score function produces fp32 probs and a [T,E] routing
// map; with sigmoid scoring an fp32 expert bias shifts the choice only.
// §8: with a capacity factor each expert keeps at most `capacity` tokens,
// chosen by position (here: the earliest tokens), and the dropped entries
// leave both the map and the probs.
//
// Kernels, in launch order:
//   router_logits_ring     bf16 x: x w^T on bf16 MFMA with the fp32 weight split
//                          exactly into three bf16 parts (fp32-accurate), both
//                          operands streamed through a ring of LDS stages,
//                          split over h into partial sums (more workgroups)
//   router_logits_simt     fp32 x (or h not a multiple of 16): fp32 FMA, LDS-tiled
//   router_topk_row_kernel E <= 256: one 16-lane row per token (16 tokens per
//                          workgroup at once): logits = partials summed in a
//                          fixed order (+ b), scores, K rounds of an argmax over
//                          the row (DPP exchanges), probs, map, per-block counts
//   router_topk_kernel     E > 256: the same with one wave per token
//   count_scan_kernel      per-expert prefix over blocks and tokens_per_expert;
//                          with a capacity, also clears the entries ranked >= capacity
#include <algorithm>
#include <cmath>
#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

// ------------------------------------------------------------- gating linear
// Tile: 64 tokens x 64 experts per 256-thread workgroup, 4x4 outputs per
// thread, k-slabs of 32 staged through LDS (x transposed so that a thread
// reads its 4 tokens with one 16-byte LDS load).
constexpr int LT = 64, LE = 64, LK = 32;

template <typename XT>
__device__ __forceinline__ float load_x(const XT* p);
template <>
__device__ __forceinline__ float load_x<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_x<uint16_t>(const uint16_t* p) { return bf16_bits_to_f32(*p); }

template <typename XT>
__global__ void __launch_bounds__(256) router_logits_simt(const XT* __restrict__ x,
                                                          const float* __restrict__ w,
                                                          float* __restrict__ logits, int64_t T,
                                                          int h, int E) {
  __shared__ float xs[LK][LT + 4];
  __shared__ float ws[LK][LE + 4];
  const int tid = threadIdx.x;
  const int tx = tid % 16;  // experts tx*4 .. +3
  const int ty = tid / 16;  // tokens  ty*4 .. +3
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * LT;
  const int e0 = blockIdx.y * LE;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < h; k0 += LK) {
    // stage: 64 rows x 32 k for x and for w; each thread moves 8 elements of each
    for (int i = tid; i < LT * LK; i += 256) {
      const int r = i / LK, c = i % LK;
      const int64_t t = t0 + r;
      const int k = k0 + c;
      xs[c][r] = (t < T && k < h) ? load_x<XT>(x + t * h + k) : 0.f;
      const int e = e0 + r;
      ws[c][r] = (e < E && k < h) ? w[static_cast<int64_t>(e) * h + k] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < LK; ++c) {
      const float4 xv = *reinterpret_cast<const float4*>(&xs[c][ty * 4]);
      const float4 wv = *reinterpret_cast<const float4*>(&ws[c][tx * 4]);
      const float xa[4] = {xv.x, xv.y, xv.z, xv.w};
      const float wa[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xa[i], wa[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) logits[t * E + e] = acc[i][j];
    }
  }
}

// ------------------------------------------------ gating linear on MFMA
// bf16 x is exact in bf16; the fp32 weight w is split exactly into
// w = hi + mid + lo, three bf16 values: hi keeps w's top 16 bits, the
// subtraction w - hi is exact (same sign and exponent), mid keeps the top 16
// bits of that remainder, and the last remainder has at most 8 significant
// bits, so lo holds it exactly.  Each product x*part is exact in fp32 and the
// MFMA accumulates in fp32: the logits have fp32 accuracy at bf16 MFMA rate.
//
// A wave owns 64 tokens x 64 experts (2x2 blocks of v_mfma_f32_32x32x16_bf16,
// three MFMAs per block per 16-wide k step); the 4 waves of a workgroup tile
// WT x WE such blocks.  blockIdx.y selects a slice of h whose partial sums go
// to their own [T, E] plane.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Split eight fp32 weights into their hi/mid/lo bf16 parts (see above),
// each part as one 8-wide bf16 MFMA operand.  A part's bf16 value is the top
// half of an fp32 word (v, then r1 = v - hi, then r2 = r1 - mid), so two
// parts are packed by one byte permute of the two words' top halves.
__device__ __forceinline__ uint32_t top_halves(float lo_elem, float hi_elem) {
  // bytes 2,3 of lo_elem then bytes 2,3 of hi_elem (selector indices 4-7 pick
  // from the first operand, 0-3 from the second)
  return __builtin_amdgcn_perm(__float_as_uint(hi_elem), __float_as_uint(lo_elem), 0x07060302u);
}
__device__ __forceinline__ void split8(const f32x4_t a, const f32x4_t b, bf16x8_t& hi,
                                       bf16x8_t& mi, bf16x8_t& lo) {
  float v[8], r1[8], r2[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[q] = a[q];
    v[q + 4] = b[q];
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    r1[q] = v[q] - __uint_as_float(__float_as_uint(v[q]) & 0xffff0000u);
    r2[q] = r1[q] - __uint_as_float(__float_as_uint(r1[q]) & 0xffff0000u);
  }
  u32x4_t h, m, l;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    h[q] = top_halves(v[2 * q], v[2 * q + 1]);
    m[q] = top_halves(r1[2 * q], r1[2 * q + 1]);
    l[q] = top_halves(r2[2 * q], r2[2 * q + 1]);
  }
  hi = __builtin_bit_cast(bf16x8_t, h);
  mi = __builtin_bit_cast(bf16x8_t, m);
  lo = __builtin_bit_cast(bf16x8_t, l);
}

// Gating linear on MFMA through a ring of LDS stages.  A wave owns 32*NI
// experts x 32*NJ tokens (NI x NJ blocks of v_mfma_f32_32x32x16_bf16, three
// MFMAs per block and k step); the 4 waves of a workgroup are WT along tokens
// x WE along experts, so a workgroup owns BT = 32*NJ*WT tokens x BE =
// 32*NI*WE experts over one slice of h, in SK-wide k slabs.  A stage holds
// one slab's x rows (BT x 2*SK bytes of bf16) and weight rows (BE x 4*SK
// bytes of fp32), filled by direct global->LDS loads, and STAGES-1 slabs
// stay in flight while one is multiplied.  Each wave reads its fragments
// from LDS and splits its fp32 weight fragments into their three bf16 parts
// in registers: with NI = 1 a wave splits one fragment per k step for four
// token blocks, which keeps the split's VALU work under the MFMA time.
// blockIdx.y selects a slice of h whose partial sums go to their own [T, E]
// plane.
template <int WT, int WE, int NI, int NJ, int STAGES, int SK>
__global__ void __launch_bounds__(256) router_logits_ring(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ w,
                                                          float* __restrict__ part, int64_t T,
                                                          int h, int E, int kchunk) {
  static_assert(WT * WE == 4, "4 waves");
  constexpr int BT = 32 * NJ * WT, BE = 32 * NI * WE;
  static_assert(SK == 32 || SK == 64, "k per slab");
  constexpr int XB = BT * SK * 2;  // x bytes per stage
  constexpr int WB = BE * SK * 4;  // weight bytes per stage
  constexpr int STAGE = XB + WB;
  constexpr int LPW = STAGE / 4096;  // 1 KB direct loads per wave per stage
  static_assert(STAGE % 4096 == 0, "whole loads per wave");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = wave / WE, we = wave % WE;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * BT;
  const int e0 = blockIdx.z * BE;
  const int kb = blockIdx.y * kchunk;
  const int nsl = (min(h, kb + kchunk) - kb) / SK;
  const uint32_t smem_base = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));
  // this lane's sources (rows clamped in range; their results are never stored)
  const char* src[LPW];
  int step[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int o = (wave * LPW + j) * 1024 + lane * 16;
    int row, c;
    if (o < XB) {
      lds_piece<SK>(o, row, c);
      src[j] = reinterpret_cast<const char*>(x + min(t0 + row, T - 1) * h + kb + c * 8);
      step[j] = SK * 2;
    } else {
      lds_piece<2 * SK>(o - XB, row, c);
      src[j] = reinterpret_cast<const char*>(w + static_cast<int64_t>(min(e0 + row, E - 1)) * h +
                                             kb + c * 4);
      step[j] = SK * 4;
    }
  }
  auto issue = [&](int sl) {
    const uint32_t dst = smem_base + static_cast<uint32_t>((sl % STAGES) * STAGE + wave * LPW * 1024);
#pragma unroll
    for (int j = 0; j < LPW; ++j) dma16(src[j] + static_cast<int64_t>(sl) * step[j], dst + j * 1024);
  };
  f32x16_t acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int sl = 0; sl < STAGES; ++sl)
    if (sl < nsl) issue(sl);
  for (int sl = 0; sl < nsl; ++sl) {
    wait_stage<LPW, STAGES>(min(sl + STAGES - 1, nsl - 1) - sl);
    block_barrier();
    const char* st = smem + (sl % STAGES) * STAGE;
#pragma unroll
    for (int kk = 0; kk < SK / 16; ++kk) {
      bf16x8_t xb[NJ], wp[3][NI];
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        xb[j] = *reinterpret_cast<const bf16x8_t*>(
            st + lds_chunk_byte<SK>(wt * 32 * NJ + j * 32 + l32, kk * 2 + hi));
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int row = we * 32 * NI + i * 32 + l32;
        const int cw = kk * 4 + hi * 2;
        const f32x4_t a =
            *reinterpret_cast<const f32x4_t*>(st + XB + lds_chunk_byte<2 * SK>(row, cw));
        const f32x4_t b =
            *reinterpret_cast<const f32x4_t*>(st + XB + lds_chunk_byte<2 * SK>(row, cw + 1));
        split8(a, b, wp[0][i], wp[1][i], wp[2][i]);
      }
#pragma unroll
      for (int pl = 0; pl < 3; ++pl)
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wp[pl][i], xb[j], acc[i][j], 0, 0, 0);
    }
    if (sl + STAGES < nsl) {
      wait_lgkm0();
      block_barrier();  // every wave is done with this slot
      issue(sl + STAGES);
    }
  }
  // Epilogue through LDS (the ring is free once every wave is past its last
  // slab): lane holds [token l32 of block j][experts 8g + 4*(lane/32) + q of
  // block i]; the tile is written to LDS rows of BE floats (+4 of padding
  // against bank conflicts), then each plane row is stored with contiguous
  // 16-byte stores (16 lanes per 256 bytes) instead of scattered dwords.
  constexpr int OS = BE + 4;
  static_assert(BT * OS * 4 <= STAGES * STAGE, "output tile fits the ring");
  __syncthreads();
  float* ot = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int tl = wt * 32 * NJ + j * 32 + l32;
        const int el = we * 32 * NI + i * 32 + g * 8 + hi * 4;
        f32x4_t v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[i][j][g * 4 + q];
        *reinterpret_cast<f32x4_t*>(ot + tl * OS + el) = v;
      }
  __syncthreads();
  float* out = part + static_cast<int64_t>(blockIdx.y) * T * E;
  constexpr int CPR = BE / 4;  // 16-byte chunks per tile row
  const bool vec = E % 4 == 0;
  for (int c = tid; c < BT * CPR; c += 256) {
    const int rl = c / CPR, e = e0 + (c % CPR) * 4;
    const int64_t t = t0 + rl;
    if (t >= T || e >= E) continue;
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(ot + rl * OS + (c % CPR) * 4);
    if (vec) {
      *reinterpret_cast<f32x4_t*>(out + t * E + e) = v;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (e + q < E) out[t * E + e + q] = v[q];
    }
  }
}

constexpr int kMaxSplit = 8;  // partial-logit planes at most

struct MfmaPlan {
  int shape;  // 0: 256 x 32 (E <= 32), 1: 128 x 64 (E <= 64), 2: 128 x 128 tokens x experts
  int bt, be;
  int64_t gx, gz;
  int ksplit, kchunk;
};

// Workgroup tile and h-split for the MFMA gating linear: the narrowest
// expert tile that covers E (up to 128), then h split into at most 8
// partial planes of >= 128 so that about 256 workgroups (one per CU) run.
// Timed on the Switch-, Mixtral-, Qwen3- and DeepSeek-V3-shaped routers,
// more planes (two workgroups per CU) were slower or equal: the extra plane
// traffic outweighs the occupancy.
MfmaPlan mfma_plan(int64_t T, int64_t h, int64_t E) {
  MfmaPlan p;
  p.shape = E <= 32 ? 0 : E <= 64 ? 1 : 2;
  p.bt = p.shape == 0 ? 256 : 128;
  p.be = p.shape == 0 ? 32 : p.shape == 1 ? 64 : 128;
  p.gx = ceil_div(T, p.bt);
  p.gz = ceil_div(E, p.be);
  const int64_t base = p.gx * p.gz;
  int64_t ks = std::min<int64_t>(kMaxSplit, std::max<int64_t>(1, ceil_div(256, base)));
  ks = std::min<int64_t>(ks, std::max<int64_t>(1, h / 128));
  p.kchunk = static_cast<int>(ceil_div(ceil_div(h, ks), 32) * 32);
  p.ksplit = static_cast<int>(ceil_div(h, p.kchunk));
  return p;
}

bool use_mfma(const moe_route_desc* d) { return d->x_dtype == MOE_BF16 && d->h % 32 == 0; }

// ------------------------------------------------------- fixed fp32 sigmoid
// exp(y) for y <= 0 by a fixed sequence of IEEE fp32 operations, each rounded
// to nearest even with no fused multiply-add: n = rint(y*log2e); Cody-Waite
// reduction r = (y - n*C1) - n*C2 with C1 = ln2 cut to 12 significant bits
// and C2 = fp32(ln2 - C1); p = degree-7 Taylor polynomial of e^r in Horner
// form with fp32(1/k!) coefficients; result ldexp(p, n); 0 below y = -86
// (keeps every result in the fp32 normal range).
__device__ __forceinline__ float exp_fixed(float y) {
#pragma clang fp contract(off)
  const float log2e = 0x1.715476p+0f;  // fp32(1/ln 2)
  const float c1 = 0x1.62ep-1f;        // ln 2 truncated to 12 bits
  const float c2 = 0x1.0bfbe8p-15f;    // fp32(ln 2 - c1)
  const float n = rintf(y * log2e);
  const float r = (y - n * c1) - n * c2;
  float p = 0x1.a01a02p-13f;           // 1/7!
  p = p * r + 0x1.6c16c2p-10f;         // 1/6!
  p = p * r + 0x1.111112p-7f;          // 1/5!
  p = p * r + 0x1.555556p-5f;          // 1/4!
  p = p * r + 0x1.555556p-3f;          // 1/3!
  p = p * r + 0.5f;                    // 1/2!
  p = p * r + 1.0f;                    // 1/1!
  p = p * r + 1.0f;                    // 1/0!
  const float out = ldexpf(p, static_cast<int>(n));
  return (y < -86.0f) ? 0.0f : out;
}

// sigmoid(x) = 1/(1+e) for x >= 0, e/(1+e) for x < 0, with e = exp_fixed(-|x|).
__device__ __forceinline__ float sigmoid_fixed(float x) {
#pragma clang fp contract(off)
  const float e = exp_fixed(-fabsf(x));
  const float den = 1.0f + e;
  return (x >= 0.0f) ? (1.0f / den) : (e / den);
}

// sqrt(softplus(x)) by a fixed fp32 sequence: softplus(x) = x for x > 20,
// else max(x, 0) + log1p(e) with e = exp_fixed(-|x|); log1p(u), 0 <= u <= 1,
// is 2*atanh(s) with s = u/(2+u) <= 1/3: (2*s) * q, q the degree-7 Horner
// polynomial in s*s with fp32(1/(2j+1)) coefficients; then the correctly
// rounded square root.
__device__ __forceinline__ float sqrtsoftplus_fixed(float x) {
#pragma clang fp contract(off)
  const float e = exp_fixed(-fabsf(x));
  const float s = e / (2.0f + e);
  const float s2 = s * s;
  float q = 0x1.111112p-4f;          // 1/15
  q = q * s2 + 0x1.3b13b2p-4f;       // 1/13
  q = q * s2 + 0x1.745d18p-4f;       // 1/11
  q = q * s2 + 0x1.c71c72p-4f;       // 1/9
  q = q * s2 + 0x1.24924ap-3f;       // 1/7
  q = q * s2 + 0x1.99999ap-3f;       // 1/5
  q = q * s2 + 0x1.555556p-2f;       // 1/3
  q = q * s2 + 1.0f;                 // 1/1
  const float l1p = (2.0f * s) * q;
  const float sp = (x > 20.0f) ? x : (fmaxf(x, 0.0f) + l1p);
  return sqrtf(sp);  // correctly rounded (no fast-math flags)
}

// --------------------------------------------------------------- top-k
// (value descending, index ascending) is a strict total order on non-NaN
// keys, so a butterfly reduction gives every lane the same winner.
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  if (ai < 0) return false;
  if (bi < 0) return true;
  return av > bv || (av == bv && ai < bi);
}

template <int EPL>
__global__ void __launch_bounds__(256) router_topk_kernel(
    const float* __restrict__ part, int nsplit, const float* __restrict__ bias,
    const float* __restrict__ expert_bias, int64_t T, int E, int K, int score, int pre_softmax,
    float* __restrict__ logits_out, float* __restrict__ scores_out, float* __restrict__ probs,
    uint8_t* __restrict__ rmap, int32_t* __restrict__ hist) {
  __shared__ int cnt[kMaxExperts];
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  constexpr int kTokPerWave = kCountBlock / 4;
  // Phase 1: logits of all of this wave's tokens (every partial plane is
  // loaded before any is summed; planes are summed in order, then the bias).
  float lt[kTokPerWave][EPL];
  const int64_t tw = static_cast<int64_t>(blockIdx.x) * kCountBlock + wave * kTokPerWave;
#pragma unroll
  for (int it = 0; it < kTokPerWave; ++it) {
    const int64_t t = min(tw + it, T - 1);  // clamped; tokens past T are skipped below
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = min(lane + 64 * j, E - 1);
      const int64_t idx = t * E + e;
      float pv[kMaxSplit];
#pragma unroll
      for (int sp = 0; sp < kMaxSplit; ++sp) pv[sp] = sp < nsplit ? part[sp * T * E + idx] : 0.f;
      float v = pv[0];
#pragma unroll
      for (int sp = 1; sp < kMaxSplit; ++sp)
        if (sp < nsplit) v += pv[sp];
      if (bias) v += bias[e];
      lt[it][j] = v;
    }
  }
#pragma unroll
  for (int it = 0; it < kTokPerWave; ++it) {
    const int64_t t = tw + it;
    if (t >= T) break;  // wave-uniform
    float l[EPL], s[EPL], key[EPL];
    bool valid[EPL], taken[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      valid[j] = e < E;
      taken[j] = false;
      l[j] = valid[j] ? lt[it][j] : -INFINITY;
      if (valid[j] && logits_out) logits_out[t * E + e] = l[j];
    }
    if (score == MOE_SCORE_SOFTMAX) {
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < EPL; ++j) m = fmaxf(m, l[j]);
      m = wave_max(m);
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        s[j] = valid[j] ? expf(l[j] - m) : 0.f;
        sum += s[j];
      }
      sum = wave_sum(sum);
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        s[j] = s[j] / sum;
        key[j] = l[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        s[j] = valid[j] ? (score == MOE_SCORE_SIGMOID ? sigmoid_fixed(l[j]) : sqrtsoftplus_fixed(l[j]))
                        : 0.f;
        key[j] = (valid[j] && expert_bias) ? s[j] + expert_bias[lane + 64 * j] : s[j];
      }
    }
    float top_logit = 0.f;
    for (int k = 0; k < K; ++k) {
      float bv = 0.f;
      int bi = -1;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = lane + 64 * j;
        if (valid[j] && !taken[j] && better(key[j], e, bv, bi)) {
          bv = key[j];
          bi = e;
        }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      bi = __shfl(bi, 0, 64);
      if (k == 0) top_logit = __shfl(bv, 0, 64);
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (lane + 64 * j == bi) taken[j] = true;
    }
    float p[EPL];
    if (score == MOE_SCORE_SOFTMAX && pre_softmax) {
#pragma unroll
      for (int j = 0; j < EPL; ++j) p[j] = taken[j] ? s[j] : 0.f;
    } else if (score == MOE_SCORE_SOFTMAX) {
      // softmax over the K chosen logits; the first winner holds their maximum
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        p[j] = taken[j] ? expf(l[j] - top_logit) : 0.f;
        sum += p[j];
      }
      sum = wave_sum(sum);
#pragma unroll
      for (int j = 0; j < EPL; ++j) p[j] = p[j] / sum;
    } else {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < EPL; ++j) sum += taken[j] ? s[j] : 0.f;
      sum = wave_sum(sum) + 1e-20f;
#pragma unroll
      for (int j = 0; j < EPL; ++j) p[j] = taken[j] ? s[j] / sum : 0.f;
    }
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      if (!valid[j]) continue;
      probs[t * E + e] = p[j];
      rmap[t * E + e] = taken[j] ? 1 : 0;
      if (scores_out) scores_out[t * E + e] = s[j];
      if (taken[j]) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    hist[static_cast<int64_t>(e) * gridDim.x + blockIdx.x] = cnt[e];
}

// Top-k with one 16-lane row per token (E <= 256): a workgroup's 16 rows
// are its 16 tokens, all handled at once; lane r of a row holds experts
// r*VPL .. r*VPL+VPL-1 (contiguous, so a row reads a token's logits with
// vector loads).  Reductions over the row are DPP exchanges within the
// 16-lane row (swap neighbours, swap pairs, half-row mirror, row mirror),
// after which every lane of the row holds the same result.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i within each 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15-i within the row

__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  return fmaxf(v, dpp_f<kDppMirror>(v));
}
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  return v + dpp_f<kDppMirror>(v);
}
template <int CTRL>
__device__ __forceinline__ void arg_step(float& bv, int& bi) {
  const float ov = dpp_f<CTRL>(bv);
  const int oi = dpp_i<CTRL>(bi);
  // better(ov, oi, bv, bi) as selects
  const bool c = oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi));
  bv = c ? ov : bv;
  bi = c ? oi : bi;
}

template <int VPL>
__global__ void __launch_bounds__(256) router_topk_row_kernel(
    const float* __restrict__ part, int nsplit, const float* __restrict__ bias,
    const float* __restrict__ expert_bias, int64_t T, int E, int K, int score, int pre_softmax,
    float* __restrict__ logits_out, float* __restrict__ scores_out, float* __restrict__ probs,
    uint8_t* __restrict__ rmap, int32_t* __restrict__ hist, int aligned) {
  static_assert(kCountBlock == 16, "one token per 16-lane row");
  __shared__ int cnt[16 * VPL];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int r = threadIdx.x & 15;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kCountBlock + threadIdx.x / 16;
  const int e0 = r * VPL;
  if (t < T) {  // uniform over the row
    bool valid[VPL];
    float l[VPL], s[VPL], key[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      valid[j] = e0 + j < E;
    }
    // logits: the partial planes summed in plane order, then the bias
    const int64_t row = t * E;
    // groups of 4 experts as vectors: E % 4 == 0 and every array 16-byte
    // aligned (the map 4-byte aligned)
    const bool vec = (VPL % 4 == 0) && (E % 4 == 0) && aligned;
    auto load_plane = [&](int sp, float* v) {
      const float* src = part + static_cast<int64_t>(sp) * T * E + row;
      if (vec) {  // E % 4 == 0: a group of 4 is wholly in or out of the row
#pragma unroll
        for (int j = 0; j < VPL; j += 4) {
          const float4 q = valid[j] ? *reinterpret_cast<const float4*>(src + e0 + j)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
          v[j] = q.x;
          v[j + 1] = q.y;
          v[j + 2] = q.z;
          v[j + 3] = q.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < VPL; ++j) v[j] = valid[j] ? src[e0 + j] : 0.f;
      }
    };
    float acc[VPL];
    load_plane(0, acc);
    constexpr int kInFlight = VPL <= 4 ? 7 : VPL <= 8 ? 4 : 2;  // planes loaded together
    for (int sp0 = 1; sp0 < nsplit; sp0 += kInFlight) {
      float pv[kInFlight][VPL];
#pragma unroll
      for (int u = 0; u < kInFlight; ++u)
        if (sp0 + u < nsplit) load_plane(sp0 + u, pv[u]);
#pragma unroll
      for (int u = 0; u < kInFlight; ++u)
        if (sp0 + u < nsplit)
#pragma unroll
          for (int j = 0; j < VPL; ++j) acc[j] += pv[u][j];
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      float v = acc[j];
      if (bias && valid[j]) v += bias[e0 + j];
      l[j] = valid[j] ? v : -INFINITY;
    }
    if (score == MOE_SCORE_SOFTMAX) {
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < VPL; ++j) m = fmaxf(m, l[j]);
      m = row_max(m);
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        s[j] = valid[j] ? expf(l[j] - m) : 0.f;
        sum += s[j];
      }
      sum = row_sum(sum);
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        s[j] = s[j] / sum;
        key[j] = l[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        s[j] = valid[j] ? (score == MOE_SCORE_SIGMOID ? sigmoid_fixed(l[j]) : sqrtsoftplus_fixed(l[j]))
                        : 0.f;
        key[j] = (valid[j] && expert_bias) ? s[j] + expert_bias[e0 + j] : s[j];
      }
    }
    // K rounds of argmax, branch-free: bit j of `tk` marks expert e0 + j taken.
    // Within a lane experts are scanned in ascending order, so a later equal
    // key never displaces the earlier one.
    float top_logit = 0.f;
    uint32_t tk = 0;
    for (int k = 0; k < K; ++k) {
      float bv = 0.f;
      int bi = -1;
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const bool c = valid[j] && !((tk >> j) & 1u) && (bi < 0 || key[j] > bv);
        bv = c ? key[j] : bv;
        bi = c ? e0 + j : bi;
      }
      arg_step<kDppXor1>(bv, bi);
      arg_step<kDppXor2>(bv, bi);
      arg_step<kDppHalfMirror>(bv, bi);
      arg_step<kDppMirror>(bv, bi);
      if (k == 0) top_logit = bv;
      const uint32_t d = static_cast<uint32_t>(bi - e0);
      tk |= d < static_cast<uint32_t>(VPL) ? 1u << d : 0u;
    }
    bool taken[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) taken[j] = (tk >> j) & 1u;
    float p[VPL];
    if (score == MOE_SCORE_SOFTMAX && pre_softmax) {
#pragma unroll
      for (int j = 0; j < VPL; ++j) p[j] = taken[j] ? s[j] : 0.f;
    } else if (score == MOE_SCORE_SOFTMAX) {
      // softmax over the K chosen logits; the first winner holds their maximum
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        p[j] = taken[j] ? expf(l[j] - top_logit) : 0.f;
        sum += p[j];
      }
      sum = row_sum(sum);
#pragma unroll
      for (int j = 0; j < VPL; ++j) p[j] = p[j] / sum;
    } else {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < VPL; ++j) sum += taken[j] ? s[j] : 0.f;
      sum = row_sum(sum) + 1e-20f;
#pragma unroll
      for (int j = 0; j < VPL; ++j) p[j] = taken[j] ? s[j] / sum : 0.f;
    }
    if (vec) {  // whole groups of 4: 16-byte stores (4 bytes for the map)
#pragma unroll
      for (int j = 0; j < VPL; j += 4) {
        if (!valid[j]) continue;
        *reinterpret_cast<float4*>(probs + row + e0 + j) = make_float4(p[j], p[j + 1], p[j + 2], p[j + 3]);
        *reinterpret_cast<uint32_t*>(rmap + row + e0 + j) =
            (taken[j] ? 1u : 0u) | (taken[j + 1] ? 1u << 8 : 0u) | (taken[j + 2] ? 1u << 16 : 0u) |
            (taken[j + 3] ? 1u << 24 : 0u);
        if (logits_out)
          *reinterpret_cast<float4*>(logits_out + row + e0 + j) = make_float4(l[j], l[j + 1], l[j + 2], l[j + 3]);
        if (scores_out)
          *reinterpret_cast<float4*>(scores_out + row + e0 + j) = make_float4(s[j], s[j + 1], s[j + 2], s[j + 3]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        if (!valid[j]) continue;
        probs[row + e0 + j] = p[j];
        rmap[row + e0 + j] = taken[j] ? 1 : 0;
        if (logits_out) logits_out[row + e0 + j] = l[j];
        if (scores_out) scores_out[row + e0 + j] = s[j];
      }
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (valid[j] && taken[j]) atomicAdd(&cnt[e0 + j], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    hist[static_cast<int64_t>(e) * gridDim.x + blockIdx.x] = cnt[e];
}

// ------------------------------------------------- capacity mask per expert
// One workgroup per expert e: the capacity mask of column e is the first
// `cap` of the T tokens by (key descending, token ascending), with key =
// the routing prob (probs policy) or the map entry (position policy).  The
// cap-th largest key v is found by a radix select over the 31 magnitude
// bits (4 passes of 8 bits, LDS histograms); then every token with key > v
// is in the mask, and of the tokens with key == v the earliest `need`
// ones (an ordered block scan over the tokens).  The final map is the mask
// (padding to capacity) or map AND mask; final probs = probs * final map;
// tokens_per_expert[e] = column sum of the final map.
__device__ __forceinline__ uint32_t cap_key(const float* probs, const uint8_t* rmap, int64_t idx,
                                            int policy) {
  return policy == MOE_DROP_PROBS ? (__float_as_uint(probs[idx]) & 0x7fffffffu)
                                  : (rmap[idx] ? 1u : 0u);
}

__global__ void __launch_bounds__(256) router_capacity_kernel(int64_t T, int E, int64_t cap,
                                                              int policy, int pad,
                                                              float* __restrict__ probs,
                                                              uint8_t* __restrict__ rmap,
                                                              int32_t* __restrict__ counts) {
  __shared__ int hist[256];
  __shared__ int64_t scratch[4];
  __shared__ uint32_t s_digit;
  __shared__ int64_t s_rank;
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  // rank (1-based) of the wanted key among keys sharing the prefix so far
  int64_t rank = cap;
  uint32_t prefix = 0, pmask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int64_t t = tid; t < T; t += 256) {
      const uint32_t k = cap_key(probs, rmap, t * E + e, policy);
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid == 0) {
      // walk digits from the top until the count reaches the rank
      int64_t acc = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (acc + hist[d] >= rank) break;
        acc += hist[d];
      }
      s_digit = static_cast<uint32_t>(d);
      s_rank = rank - acc;
    }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= 255u << shift;
    rank = s_rank;
    __syncthreads();
  }
  const uint32_t v = prefix;  // the cap-th largest key
  // `rank` = how many tokens with key == v belong to the mask (earliest first)
  const int64_t need = rank;
  int64_t seen = 0;  // tokens with key == v in earlier chunks
  int64_t kept = 0;
  for (int64_t t0 = 0; t0 < T; t0 += 256) {
    const int64_t t = t0 + tid;
    uint32_t k = 0;
    bool eq = false;
    if (t < T) {
      k = cap_key(probs, rmap, t * E + e, policy);
      eq = k == v;
    }
    int64_t tot;
    const int64_t before = seen + block_exclusive_scan256(eq ? 1 : 0, scratch, &tot);
    seen += tot;
    if (t < T) {
      const bool in_mask = k > v || (eq && before < need);
      const int64_t idx = t * E + e;
      const bool routed = rmap[idx] != 0;
      const bool fin = pad ? in_mask : (routed && in_mask);
      if (routed && !fin) {  // dropped
        rmap[idx] = 0;
        probs[idx] = 0.f;
      } else if (!routed && fin) {  // padding (its prob is already 0)
        rmap[idx] = 1;
      }
      kept += fin ? 1 : 0;
    }
  }
  int64_t total;
  block_exclusive_scan256(kept, scratch, &total);
  if (tid == 0) counts[e] = static_cast<int32_t>(total);
}

// ------------------------------------------- load-balancing loss value
// Pass 1: workgroup b handles tokens [64b, 64b+64): per token the score row
// sum (sigmoid-type scores are normalised per token; softmax rows are used
// as they are), then each thread accumulates its experts' normalised scores
// over the 64 tokens in token order into partial[b][e].  Pass 2 (one
// workgroup): P[e] = sum of the partials in block order / T, term[e] =
// n_e * P[e], loss = E / (T*K) * sum_e term[e] by a fixed-order tree.
constexpr int kAuxTok = 64;

__global__ void __launch_bounds__(256) aux_partial_kernel(const float* __restrict__ scores,
                                                          int64_t T, int E, int normalise,
                                                          float* __restrict__ partial) {
  __shared__ float inv[kAuxTok];
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kAuxTok;
  const int nt = static_cast<int>(min(static_cast<int64_t>(kAuxTok), T - t0));
  for (int tl = wave; tl < kAuxTok; tl += 4) {
    float sum = 0.f;
    if (normalise && tl < nt)
      for (int e = lane; e < E; e += 64) sum += scores[(t0 + tl) * E + e];
    sum = wave_sum(sum);
    if (lane == 0) inv[tl] = normalise ? 1.0f / (sum + 1e-20f) : 1.0f;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    float acc = 0.f;
    for (int tl = 0; tl < nt; ++tl) acc += scores[(t0 + tl) * E + e] * inv[tl];
    partial[static_cast<int64_t>(blockIdx.x) * E + e] = acc;
  }
}

__global__ void __launch_bounds__(256) aux_final_kernel(const float* __restrict__ partial,
                                                        int64_t nblk, int64_t T, int E, int K,
                                                        const int32_t* __restrict__ counts,
                                                        float* __restrict__ loss) {
  __shared__ float red[256];
  float term = 0.f;
  for (int e = threadIdx.x; e < E; e += 256) {
    float P = 0.f;
    for (int64_t b = 0; b < nblk; ++b) P += partial[b * E + e];
    term += static_cast<float>(counts[e]) * (P / static_cast<float>(T));
  }
  red[threadIdx.x] = term;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0)
    loss[0] = red[0] * (static_cast<float>(E) / (static_cast<float>(T) * static_cast<float>(K)));
}

// ------------------------------------------------- expert-bias controller
__global__ void __launch_bounds__(256) accumulate_tokens_kernel(int E,
                                                                const int32_t* __restrict__ tpe,
                                                                int64_t* __restrict__ local) {
  for (int e = blockIdx.x * 256 + threadIdx.x; e < E; e += gridDim.x * 256) local[e] += tpe[e];
}

// bias[e] += sign(S - E*c[e]) * rate with S = sum of the counts (exact
// integer comparison of the count with the mean); optionally zero the counts.
__global__ void __launch_bounds__(256) update_bias_kernel(int E, int64_t* __restrict__ local,
                                                          float* __restrict__ bias, float rate,
                                                          int reset) {
  __shared__ int64_t scratch[4];
  constexpr int PER = kMaxExperts / 256;
  int64_t c[PER], sum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = threadIdx.x * PER + j;
    c[j] = e < E ? local[e] : 0;
    sum += c[j];
  }
  int64_t S;
  block_exclusive_scan256(sum, scratch, &S);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = threadIdx.x * PER + j;
    if (e >= E) continue;
    const int64_t d = S - static_cast<int64_t>(E) * c[j];
    const float sgn = d > 0 ? 1.0f : (d < 0 ? -1.0f : 0.0f);
    bias[e] = bias[e] + sgn * rate;
    if (reset) local[e] = 0;
  }
}

struct TopkArgs {
  const float* part;
  int nsplit;
  const float* bias;
  const float* expert_bias;
  int64_t T;
  int E, K, score, pre;
  float *logits_out, *scores, *probs;
  uint8_t* map;
  int32_t* hist;
};

template <int EPL>
void launch_topk(int64_t nblk, hipStream_t s, const TopkArgs& a) {
  hipLaunchKernelGGL(router_topk_kernel<EPL>, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s,
                     a.part, a.nsplit, a.bias, a.expert_bias, a.T, a.E, a.K, a.score, a.pre,
                     a.logits_out, a.scores, a.probs, a.map, a.hist);
}

template <int VPL>
void launch_topk_row(int64_t nblk, hipStream_t s, const TopkArgs& a) {
  const uintptr_t f = reinterpret_cast<uintptr_t>(a.part) | reinterpret_cast<uintptr_t>(a.logits_out) |
                      reinterpret_cast<uintptr_t>(a.scores) | reinterpret_cast<uintptr_t>(a.probs);
  const int aligned = (f % 16 == 0) && (reinterpret_cast<uintptr_t>(a.map) % 4 == 0);
  hipLaunchKernelGGL(router_topk_row_kernel<VPL>, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s,
                     a.part, a.nsplit, a.bias, a.expert_bias, a.T, a.E, a.K, a.score, a.pre,
                     a.logits_out, a.scores, a.probs, a.map, a.hist, aligned);
}

size_t logits_ws_bytes(const moe_route_desc* d) {
  const int64_t planes = use_mfma(d) ? mfma_plan(d->T, d->h, d->E).ksplit : 1;
  return align_up(static_cast<size_t>(planes * d->T * d->E) * sizeof(float), 256);
}

// max(ceil(T*K*cf/E), min_capacity), or -1 when dropless (cf <= 0)
int64_t raw_capacity(const moe_route_desc* d) {
  if (!(d->capacity_factor > 0.f)) return -1;
  const double ratio = static_cast<double>(d->T) * static_cast<double>(d->K) *
                       static_cast<double>(d->capacity_factor) / static_cast<double>(d->E);
  int64_t cap = static_cast<int64_t>(std::ceil(ratio));
  if (cap < d->min_capacity) cap = d->min_capacity;
  return cap;
}

// capacity that can drop anything, or -1 (dropless, or capacity >= T)
int64_t capacity_of(const moe_route_desc* d) {
  const int64_t cap = raw_capacity(d);
  return cap >= d->T ? -1 : cap;
}

moe_status validate(const moe_route_desc* d) {
  MOE_REQUIRE(d != nullptr, MOE_ERR_ARG, "moe_route: desc is NULL");
  MOE_REQUIRE(d->T >= 0 && d->T < (int64_t(1) << 31), MOE_ERR_ARG, "moe_route: T=%lld out of range",
              (long long)d->T);
  MOE_REQUIRE(d->E >= 1 && d->E <= kMaxExperts, MOE_ERR_ARG, "moe_route: E=%lld not in [1,%lld]",
              (long long)d->E, (long long)kMaxExperts);
  MOE_REQUIRE(d->K >= 1 && d->K <= d->E && d->K <= kMaxTopK, MOE_ERR_ARG,
              "moe_route: K=%lld must be in [1, min(E, %lld)]", (long long)d->K,
              (long long)kMaxTopK);
  MOE_REQUIRE(d->h >= 1 && d->h % 8 == 0, MOE_ERR_UNSUPPORTED,
              "moe_route: h=%lld must be a positive multiple of 8", (long long)d->h);
  MOE_REQUIRE(d->x_dtype == MOE_F32 || d->x_dtype == MOE_BF16, MOE_ERR_ARG,
              "moe_route: bad x_dtype %d", d->x_dtype);
  MOE_REQUIRE(d->score == MOE_SCORE_SOFTMAX || d->score == MOE_SCORE_SIGMOID ||
                  d->score == MOE_SCORE_SQRTSOFTPLUS,
              MOE_ERR_ARG, "moe_route: bad score %d", d->score);
  MOE_REQUIRE(d->drop_policy == MOE_DROP_POSITION || d->drop_policy == MOE_DROP_PROBS, MOE_ERR_ARG,
              "moe_route: bad drop_policy %d", d->drop_policy);
  MOE_REQUIRE(d->min_capacity >= 0, MOE_ERR_ARG, "moe_route: min_capacity < 0");
  MOE_REQUIRE(static_cast<int64_t>(d->T) * d->E < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED,
              "moe_route: T*E too large");
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_route_workspace_size(const moe_route_desc* d) {
  if (validate(d) != MOE_OK || d->T == 0) return 0;
  return logits_ws_bytes(d) + count_ws_bytes(d->T, d->E);
}

extern "C" int64_t moe_route_capacity(const moe_route_desc* d) {
  if (validate(d) != MOE_OK) return -1;
  return capacity_of(d);
}

extern "C" int64_t moe_max_rows(const moe_route_desc* d) {
  if (validate(d) != MOE_OK) return -1;
  const int64_t tk = d->T * d->K;
  const int64_t raw = raw_capacity(d);
  if (raw >= 0 && d->pad_to_capacity) return std::min(raw, d->T) * d->E;  // every expert padded
  const int64_t cap = capacity_of(d);
  return cap < 0 ? tk : std::min(tk, cap * d->E);
}

namespace moe {
namespace {

// moe_route's body.  *counted (if given) is set to the per-block offsets of
// the final map (block-major [nblk, E], the counting pass's blkoff) when the
// path leaves them there (position policy or nothing dropped), else NULL.
moe_status route_impl(const moe_route_desc* d, const void* x, const float* w_router,
                      const float* b_router, const float* expert_bias, const float* logits_in,
                      float* logits_out, float* scores_out, float* probs, uint8_t* routing_map,
                      int32_t* tokens_per_expert, void* workspace, size_t workspace_bytes,
                      hipStream_t s, const int32_t** counted) {
  if (counted) *counted = nullptr;
  moe_status st = validate(d);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(tokens_per_expert, MOE_ERR_ARG, "moe_route: tokens_per_expert is required");
  MOE_REQUIRE(expert_bias == nullptr || d->score != MOE_SCORE_SOFTMAX, MOE_ERR_UNSUPPORTED,
              "moe_route: expert_bias is defined for sigmoid and sqrtsoftplus scoring only");
  const int64_t T = d->T, E = d->E;
  if (T == 0) {  // [0,E] tensors may be NULL
    launch_fill_i32(tokens_per_expert, E, 0, s);
    return check_launch("moe_route(T=0)");
  }
  MOE_REQUIRE(probs && routing_map, MOE_ERR_ARG, "moe_route: probs and routing_map are required");
  MOE_REQUIRE(logits_in || (x && w_router), MOE_ERR_ARG,
              "moe_route: x and w_router are required unless logits_in is given");
  const size_t need = moe_route_workspace_size(d);
  MOE_REQUIRE(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE,
              "moe_route: workspace of %zu bytes given, %zu needed", workspace_bytes, need);

  char* ws = static_cast<char*>(workspace);
  float* part_ws = reinterpret_cast<float*>(ws);
  const int64_t nblk = ceil_div(T, kCountBlock);
  const size_t plane_bytes = align_up(static_cast<size_t>(nblk * E) * sizeof(int32_t), 256);
  int32_t* hist = reinterpret_cast<int32_t*>(ws + logits_ws_bytes(d));
  int32_t* blkoff = hist + plane_bytes / 4;

  TopkArgs ta{};
  ta.expert_bias = expert_bias;
  ta.T = T;
  ta.E = static_cast<int>(E);
  ta.K = static_cast<int>(d->K);
  ta.score = d->score;
  ta.pre = d->pre_softmax;
  ta.logits_out = logits_out;
  ta.scores = scores_out;
  ta.probs = probs;
  ta.map = routing_map;
  ta.hist = hist;
  if (logits_in) {
    ta.part = logits_in;
    ta.nsplit = 1;
    ta.bias = nullptr;  // logits_in are complete logits
  } else if (use_mfma(d)) {
    const MfmaPlan p = mfma_plan(T, d->h, E);
    const dim3 grid(static_cast<unsigned>(p.gx), static_cast<unsigned>(p.ksplit),
                    static_cast<unsigned>(p.gz));
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const int hh = static_cast<int>(d->h), Ei = static_cast<int>(E);
    if (p.shape == 0)
      hipLaunchKernelGGL((router_logits_ring<4, 1, 1, 2, 3, 32>), grid, dim3(256), 0, s, xb, w_router,
                         part_ws, T, hh, Ei, p.kchunk);
    else if (p.shape == 1)
      hipLaunchKernelGGL((router_logits_ring<2, 2, 1, 2, 3, 32>), grid, dim3(256), 0, s, xb, w_router,
                         part_ws, T, hh, Ei, p.kchunk);
    else
      hipLaunchKernelGGL((router_logits_ring<1, 4, 1, 4, 3, 32>), grid, dim3(256), 0, s, xb, w_router,
                         part_ws, T, hh, Ei, p.kchunk);
    ta.part = part_ws;
    ta.nsplit = p.ksplit;
    ta.bias = b_router;
  } else {
    dim3 grid(static_cast<unsigned>(ceil_div(T, LT)), static_cast<unsigned>(ceil_div(E, LE)));
    if (d->x_dtype == MOE_BF16)
      hipLaunchKernelGGL(router_logits_simt<uint16_t>, grid, dim3(256), 0, s,
                         static_cast<const uint16_t*>(x), w_router, part_ws, T,
                         static_cast<int>(d->h), static_cast<int>(E));
    else
      hipLaunchKernelGGL(router_logits_simt<float>, grid, dim3(256), 0, s,
                         static_cast<const float*>(x), w_router, part_ws, T,
                         static_cast<int>(d->h), static_cast<int>(E));
    ta.part = part_ws;
    ta.nsplit = 1;
    ta.bias = b_router;
  }

  const int vpl = static_cast<int>(ceil_div(E, 16));
  const int epl = static_cast<int>(ceil_div(E, 64));
  if (vpl <= 1) launch_topk_row<1>(nblk, s, ta);
  else if (vpl <= 2) launch_topk_row<2>(nblk, s, ta);
  else if (vpl <= 4) launch_topk_row<4>(nblk, s, ta);
  else if (vpl <= 8) launch_topk_row<8>(nblk, s, ta);
  else if (vpl <= 16) launch_topk_row<16>(nblk, s, ta);
  else if (epl <= 8) launch_topk<8>(nblk, s, ta);
  else launch_topk<16>(nblk, s, ta);

  const int64_t raw = raw_capacity(d);
  if (raw >= 0 && (d->drop_policy == MOE_DROP_PROBS || d->pad_to_capacity)) {
    // per-expert capacity mask (probs policy, or padding to capacity)
    if (raw >= T && !d->pad_to_capacity) {
      launch_count_scan(hist, nblk, E, -1, blkoff, tokens_per_expert, s);  // nothing dropped
      if (counted) *counted = blkoff;
    } else {
      hipLaunchKernelGGL(router_capacity_kernel, dim3(static_cast<unsigned>(E)), dim3(256), 0, s, T,
                         static_cast<int>(E), std::min(raw, T), d->drop_policy,
                         d->pad_to_capacity, probs, routing_map, tokens_per_expert);
    }
    return check_launch("moe_route");
  }
  // position policy: tokens_per_expert = min(count, capacity), then drop
  // entries ranked >= capacity
  const int64_t cap = capacity_of(d);
  launch_count_scan(hist, nblk, E, cap, blkoff, tokens_per_expert, s, T, probs, routing_map);
  if (counted) *counted = blkoff;
  return check_launch("moe_route");
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_route(const moe_route_desc* d, const void* x, const float* w_router,
                                const float* b_router, const float* expert_bias,
                                const float* logits_in, float* logits_out, float* scores_out,
                                float* probs, uint8_t* routing_map, int32_t* tokens_per_expert,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return route_impl(d, x, w_router, b_router, expert_bias, logits_in, logits_out, scores_out, probs,
                    routing_map, tokens_per_expert, workspace, workspace_bytes, as_stream(stream),
                    nullptr);
}

extern "C" size_t moe_route_permute_workspace_size(const moe_route_desc* d) {
  if (validate(d) != MOE_OK || d->T == 0) return 0;
  return align_up(moe_route_workspace_size(d), 256) + moe_permute_workspace_size(d->T, d->E);
}

extern "C" moe_status moe_route_permute(const moe_route_desc* d, const void* x, const float* w_router,
                                        const float* b_router, const float* expert_bias,
                                        const float* logits_in, float* logits_out,
                                        float* scores_out, float* probs, uint8_t* routing_map,
                                        int32_t* tokens_per_expert, int64_t max_rows,
                                        void* permuted_x, float* permuted_probs,
                                        int32_t* sorted_token, int32_t* row_id_map,
                                        int32_t* expert_offsets, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  moe_status st = validate(d);
  if (st != MOE_OK) return st;
  // the permute's arguments are checked before anything is launched
  st = permute_check(d->T, d->h, d->E, d->K, d->x_dtype, x, routing_map, probs, max_rows,
                     permuted_x, permuted_probs, sorted_token, row_id_map, expert_offsets);
  if (st != MOE_OK) return st;
  const size_t route_bytes = align_up(moe_route_workspace_size(d), 256);
  const size_t need = moe_route_permute_workspace_size(d);
  MOE_REQUIRE(d->T == 0 || (workspace && workspace_bytes >= need), MOE_ERR_WORKSPACE,
              "moe_route_permute: workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  const hipStream_t s = as_stream(stream);
  const int32_t* counted = nullptr;
  st = route_impl(d, x, w_router, b_router, expert_bias, logits_in, logits_out, scores_out, probs,
                  routing_map, tokens_per_expert, workspace, route_bytes, s, &counted);
  if (st != MOE_OK) return st;
  char* pws = d->T == 0 ? nullptr : static_cast<char*>(workspace) + route_bytes;
  return permute_impl(d->T, d->h, d->E, d->K, d->x_dtype, x, routing_map, probs, max_rows,
                      permuted_x, permuted_probs, sorted_token, row_id_map, expert_offsets, pws,
                      d->T == 0 ? 0 : workspace_bytes - route_bytes, s, counted,
                      counted ? tokens_per_expert : nullptr);
}


extern "C" size_t moe_aux_loss_workspace_size(int64_t T, int64_t E) {
  if (T <= 0 || E <= 0 || E > kMaxExperts) return 0;
  return align_up(static_cast<size_t>(ceil_div(T, kAuxTok) * E) * sizeof(float), 256);
}

extern "C" moe_status moe_router_aux_loss(int64_t T, int64_t E, int64_t K, int32_t score,
                                          const float* scores, const int32_t* tokens_per_expert,
                                          float* loss, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  MOE_REQUIRE(T >= 0 && T < (int64_t(1) << 31), MOE_ERR_ARG, "moe_router_aux_loss: T out of range");
  MOE_REQUIRE(E >= 1 && E <= kMaxExperts, MOE_ERR_ARG, "moe_router_aux_loss: E=%lld not in [1,%lld]",
              (long long)E, (long long)kMaxExperts);
  MOE_REQUIRE(K >= 1 && K <= E, MOE_ERR_ARG, "moe_router_aux_loss: bad K=%lld", (long long)K);
  MOE_REQUIRE(score == MOE_SCORE_SOFTMAX || score == MOE_SCORE_SIGMOID ||
                  score == MOE_SCORE_SQRTSOFTPLUS,
              MOE_ERR_ARG, "moe_router_aux_loss: bad score %d", score);
  MOE_REQUIRE(T * E < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED, "moe_router_aux_loss: T*E too large");
  MOE_REQUIRE(loss && tokens_per_expert, MOE_ERR_ARG, "moe_router_aux_loss: NULL output or counts");
  const hipStream_t s = as_stream(stream);
  if (T == 0) {
    launch_fill_i32(reinterpret_cast<int32_t*>(loss), 1, 0, s);  // 0.0f
    return check_launch("moe_router_aux_loss(T=0)");
  }
  MOE_REQUIRE(scores, MOE_ERR_ARG, "moe_router_aux_loss: scores is NULL");
  const size_t need = moe_aux_loss_workspace_size(T, E);
  MOE_REQUIRE(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE,
              "moe_router_aux_loss: workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  const int64_t nblk = ceil_div(T, kAuxTok);
  float* partial = static_cast<float*>(workspace);
  hipLaunchKernelGGL(aux_partial_kernel, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s, scores,
                     T, static_cast<int>(E), score == MOE_SCORE_SOFTMAX ? 0 : 1, partial);
  hipLaunchKernelGGL(aux_final_kernel, dim3(1), dim3(256), 0, s, partial, nblk, T,
                     static_cast<int>(E), static_cast<int>(K), tokens_per_expert, loss);
  return check_launch("moe_router_aux_loss");
}

extern "C" moe_status moe_accumulate_tokens_per_expert(int64_t E, const int32_t* tokens_per_expert,
                                                       int64_t* local_tokens_per_expert,
                                                       void* stream) {
  MOE_REQUIRE(E >= 1 && E <= kMaxExperts, MOE_ERR_ARG,
              "moe_accumulate_tokens_per_expert: E=%lld not in [1,%lld]", (long long)E,
              (long long)kMaxExperts);
  MOE_REQUIRE(tokens_per_expert && local_tokens_per_expert, MOE_ERR_ARG,
              "moe_accumulate_tokens_per_expert: NULL tensor argument");
  hipLaunchKernelGGL(accumulate_tokens_kernel, dim3(static_cast<unsigned>(ceil_div(E, 256))),
                     dim3(256), 0, as_stream(stream), static_cast<int>(E), tokens_per_expert,
                     local_tokens_per_expert);
  return check_launch("moe_accumulate_tokens_per_expert");
}

extern "C" moe_status moe_update_expert_bias(int64_t E, int64_t* local_tokens_per_expert,
                                             float* expert_bias, float update_rate, int32_t reset,
                                             void* stream) {
  MOE_REQUIRE(E >= 1 && E <= kMaxExperts, MOE_ERR_ARG,
              "moe_update_expert_bias: E=%lld not in [1,%lld]", (long long)E, (long long)kMaxExperts);
  MOE_REQUIRE(local_tokens_per_expert && expert_bias, MOE_ERR_ARG,
              "moe_update_expert_bias: NULL tensor argument");
  hipLaunchKernelGGL(update_bias_kernel, dim3(1), dim3(256), 0, as_stream(stream),
                     static_cast<int>(E), local_tokens_per_expert, expert_bias, update_rate, reset);
  return check_launch("moe_update_expert_bias");
}

// ------------------------------------------------ allocation-free variant
// moe_route_permute_noalloc takes its workspace from `scratch`, a file-scope
// device array (each GPU the library runs on holds its own copy until the
// process ends).  In host code the array's name is not a device address:
// its address on the current device comes from hipGetSymbolAddress, looked
// up once per device and kept in g_scratch_ptr.  No kernel here needs the
// workspace cleared (every word a kernel reads was written earlier in the
// same call), and calls that overlap on one GPU share the array and race.
namespace moe {
namespace {
constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static_assert(kNoAllocScratchBytes % 256 == 0, "whole 256-byte units");
}  // namespace
}  // namespace moe

static __device__ __align__(256) char scratch[moe::kNoAllocScratchBytes];

namespace moe {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(MOE_ERR_HIP, "moe_route_permute_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  MOE_REQUIRE(dev >= 0 && dev < kMaxDevices, MOE_ERR_UNSUPPORTED,
              "moe_route_permute_noalloc: device %d beyond the %d the library tracks", dev,
              kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MOE_ERR_HIP, "moe_route_permute_noalloc: hipGetSymbolAddress(scratch): %s",
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace
}  // namespace moe

extern "C" moe_status moe_route_permute_noalloc(
    const moe_route_desc* d, const void* x, const float* w_router, const float* b_router,
    const float* expert_bias, const float* logits_in, float* logits_out, float* scores_out,
    float* probs, uint8_t* routing_map, int32_t* tokens_per_expert, int64_t max_rows,
    void* permuted_x, float* permuted_probs, int32_t* sorted_token, int32_t* row_id_map,
    int32_t* expert_offsets, void* stream) {
  moe_status st = validate(d);
  if (st != MOE_OK) return st;
  const size_t need = moe_route_permute_workspace_size(d);
  MOE_REQUIRE(need <= kNoAllocScratchBytes, MOE_ERR_UNSUPPORTED,
              "moe_route_permute_noalloc: this layer needs %zu bytes of workspace, more than the "
              "%zu bytes of static scratch (use moe_route_permute with a workspace)",
              need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(&ws);
    if (st != MOE_OK) return st;
  }
  return moe_route_permute(d, x, w_router, b_router, expert_bias, logits_in, logits_out,
                           scores_out, probs, routing_map, tokens_per_expert, max_rows, permuted_x,
                           permuted_probs, sorted_token, row_id_map, expert_offsets, ws,
                           need > 0 ? kNoAllocScratchBytes : 0, stream);
}
