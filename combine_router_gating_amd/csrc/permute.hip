// Dispatch preprocess: token rows to expert-major order.
//
// Megatron Core MoE 源码路径解析 §2 and §9: before the experts, the
// dispatcher reorders token rows from sequence-major to expert-major layout;
// MoE Internals: DeepSpeed-Megatron Expert Parallel Implementation §8 lists
// the same step (permute tokens into expert order).  Rows are sorted by
// (expert ascending, token ascending), which makes the order unique.
//
// Row of an entry (t, e): expert_offsets[e] + (entries of e in earlier token
// blocks) + (entries of e earlier in t's block).  The per-block counts and
// their per-expert scan (common.hip) give the second term and each expert's
// total; every scatter workgroup scans the totals in LDS for the first term
// (workgroup 0 also stores expert_offsets) and counts the third term from
// the block's map tile in LDS.
#include "moe_internal.h"

namespace moe {
namespace {

// One workgroup per block of kCountBlock tokens, one wave per token.
// Phase 1 (per token): ballots over the map row, 64 experts at a time, give
// the token's entries in ascending expert order and their rows; the entries
// with a nonzero prob take the token's combine slots (at most K: only the
// chosen experts have nonzero probs; padding to capacity adds entries with
// prob 0, which need rows but add nothing to the combine).  Phase 2: write
// row_id_map / permuted_probs / sorted_token and copy the token row, read
// once, to each of its first kMaxTopK rows with 16-byte stores; further
// rows (padding only) are copied entry by entry.
__global__ void __launch_bounds__(256) permute_scatter_kernel(
    const uint8_t* __restrict__ map, const float* __restrict__ probs, const uint4* __restrict__ x,
    int64_t T, int E, int K, int chunks, const int32_t* __restrict__ blkoff,
    const int32_t* __restrict__ totals, int32_t* __restrict__ expert_offsets, int64_t max_rows,
    uint4* __restrict__ px, float* __restrict__ pprobs, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ row_id_map) {
  __shared__ uint8_t tile[kCountBlock][kMaxExperts];
  __shared__ int rows[kCountBlock][kMaxTopK];
  __shared__ int exps[kCountBlock][kMaxTopK];
  __shared__ float sel_probs[kCountBlock][kMaxTopK];
  __shared__ int slot_rows[kCountBlock][kMaxTopK];
  __shared__ int cnt[kCountBlock];
  __shared__ int nslot[kCountBlock];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_blk[kMaxExperts];
  __shared__ int64_t scratch[4];
  const int b = blockIdx.x;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int64_t t0 = static_cast<int64_t>(b) * kCountBlock;
  const int nt = static_cast<int>(min(static_cast<int64_t>(kCountBlock), T - t0));
  // Every global read the block needs first is issued up front (one round
  // trip): the experts' totals and this block's offsets, the map tile, and
  // (E <= 256) the probs of this wave's tokens.
  constexpr int PER = kMaxExperts / 256;
  constexpr int PC = 4;  // 64-expert chunks of probs held per token (E <= 256)
  int64_t v[PER];
  int bo[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = threadIdx.x * PER + j;
    v[j] = e < E ? totals[e] : 0;
    bo[j] = e < E ? blkoff[static_cast<int64_t>(b) * E + e] : 0;
  }
  const bool pre = E <= PC * 64;
  float pv[kCountBlock / 4][PC];
  if (pre) {
#pragma unroll
    for (int i = 0; i < kCountBlock / 4; ++i)
#pragma unroll
      for (int c = 0; c < PC; ++c) {
        const int tl = wave + 4 * i, e = c * 64 + lane;
        pv[i][c] = (tl < nt && e < E) ? probs[(t0 + tl) * E + e] : 0.f;
      }
  }
  for (int i = threadIdx.x; i < nt * E; i += blockDim.x) tile[i / E][i % E] = map[t0 * E + i] != 0;
  {  // expert offsets: exclusive scan of the totals, 4 experts per thread
    int64_t sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) sum += v[j];
    int64_t all;
    int64_t pre_sum = block_exclusive_scan256(sum, scratch, &all);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = threadIdx.x * PER + j;
      if (e < E) {
        s_off[e] = static_cast<int>(pre_sum);
        s_blk[e] = bo[j];
        if (b == 0) expert_offsets[e] = static_cast<int>(pre_sum);
      }
      pre_sum += v[j];
    }
    if (threadIdx.x == 0) {
      s_off[E] = static_cast<int>(all);
      if (b == 0) expert_offsets[E] = static_cast<int>(all);
    }
  }
  __syncthreads();

  // row of entry (token tl of this block, expert e)
  auto row_of = [&](int tl, int e) {
    int prior = 0;
    for (int u = 0; u < tl; ++u) prior += tile[u][e];
    return s_off[e] + s_blk[e] + prior;
  };
  const uint64_t below = (uint64_t(1) << lane) - 1;

#pragma unroll
  for (int i = 0; i < kCountBlock / 4; ++i) {
    const int tl = wave + 4 * i;
    if (tl >= nt) break;  // wave-uniform
    const int64_t t = t0 + tl;
    int base = 0, ks = 0;
    for (int c0 = 0; c0 < E; c0 += 64) {
      const int e = c0 + lane;
      const bool set = e < E && tile[tl][e];
      float pr = 0.f;
      if (pre) {
#pragma unroll
        for (int c = 0; c < PC; ++c)
          if (c * 64 == c0) pr = pv[i][c];
      } else if (set) {
        pr = probs[t * E + e];
      }
      const bool nz = set && pr != 0.f;
      const uint64_t mask = __ballot(set);
      const uint64_t nzmask = __ballot(nz);
      if (set) {
        const int r = row_of(tl, e);
        const int j = base + __popcll(mask & below);
        if (j < kMaxTopK) {
          rows[tl][j] = r;
          exps[tl][j] = e;
          sel_probs[tl][j] = pr;
        }
        if (nz) {
          const int k = ks + __popcll(nzmask & below);
          if (k < K) slot_rows[tl][k] = r;
        }
      }
      base += __popcll(mask);
      ks += __popcll(nzmask);
    }
    if (lane == 0) {
      cnt[tl] = base;
      nslot[tl] = min(ks, K);
    }
  }
  __syncthreads();

  for (int tl = wave; tl < nt; tl += 4) {
    const int64_t t = t0 + tl;
    const int n_all = cnt[tl];
    const int n = min(n_all, kMaxTopK);
    const int ns = nslot[tl];
    if (lane < K) row_id_map[t * K + lane] = lane < ns ? slot_rows[tl][lane] : -1;
    if (lane < n) {
      const int r = rows[tl][lane];
      if (r < max_rows) {
        pprobs[r] = sel_probs[tl][lane];
        sorted_token[r] = static_cast<int32_t>(t);
      }
    }
    const uint4* src = x + t * chunks;
    if (px) {
      for (int i = lane; i < chunks; i += 64) {
        const uint4 v = src[i];
        for (int k = 0; k < n; ++k) {
          const int r = rows[tl][k];
          if (r < max_rows) px[static_cast<int64_t>(r) * chunks + i] = v;
        }
      }
    }
    if (n_all > kMaxTopK) {  // padding entries past the first kMaxTopK
      int base = 0;
      for (int c0 = 0; c0 < E; c0 += 64) {
        const int e = c0 + lane;
        const bool set = e < E && tile[tl][e];
        const uint64_t mask = __ballot(set);
        const int j = base + __popcll(mask & below);
        const int r = (set && j >= kMaxTopK) ? row_of(tl, e) : -1;
        if (r >= 0 && r < max_rows) {
          pprobs[r] = probs[t * E + e];
          sorted_token[r] = static_cast<int32_t>(t);
        }
        uint64_t todo = __ballot(r >= 0 && r < max_rows);
        while (todo) {
          const int src_lane = __builtin_ctzll(todo);
          todo &= todo - 1;
          const int rr = __shfl(r, src_lane, 64);
          if (px)
            for (int i = lane; i < chunks; i += 64) px[static_cast<int64_t>(rr) * chunks + i] = src[i];
        }
        base += __popcll(mask);
      }
    }
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_permute_workspace_size(int64_t T, int64_t E) {
  if (T <= 0 || E <= 0 || E > kMaxExperts) return 0;
  return count_ws_bytes(T, E);
}

namespace moe {

moe_status permute_check(int64_t T, int64_t h, int64_t E, int64_t K, int32_t dtype, const void* x,
                         const uint8_t* routing_map, const float* probs, int64_t max_rows,
                         const void* permuted_x, const float* permuted_probs,
                         const int32_t* sorted_token, const int32_t* row_id_map,
                         const int32_t* expert_offsets) {
  MOE_REQUIRE(T >= 0 && T < (int64_t(1) << 31), MOE_ERR_ARG, "moe_permute: T out of range");
  MOE_REQUIRE(E >= 1 && E <= kMaxExperts, MOE_ERR_ARG, "moe_permute: E=%lld not in [1,%lld]",
              (long long)E, (long long)kMaxExperts);
  MOE_REQUIRE(K >= 1 && K <= E && K <= kMaxTopK, MOE_ERR_ARG, "moe_permute: bad K=%lld",
              (long long)K);
  MOE_REQUIRE(h >= 1 && h % 8 == 0, MOE_ERR_UNSUPPORTED, "moe_permute: h=%lld must be a multiple of 8",
              (long long)h);
  MOE_REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, MOE_ERR_ARG, "moe_permute: bad dtype %d", dtype);
  MOE_REQUIRE(max_rows >= 0 && max_rows < (int64_t(1) << 31), MOE_ERR_ARG,
              "moe_permute: max_rows out of range");
  MOE_REQUIRE(T * E < (int64_t(1) << 31), MOE_ERR_UNSUPPORTED, "moe_permute: T*E too large");
  MOE_REQUIRE(expert_offsets, MOE_ERR_ARG, "moe_permute: expert_offsets is required");
  if (T == 0) return MOE_OK;  // every other tensor is empty and may be NULL
  MOE_REQUIRE(routing_map && probs && row_id_map, MOE_ERR_ARG,
              "moe_permute: NULL tensor argument");
  MOE_REQUIRE(x || !permuted_x, MOE_ERR_ARG, "moe_permute: x is NULL but permuted_x is not");
  MOE_REQUIRE(max_rows == 0 || (permuted_probs && sorted_token), MOE_ERR_ARG,
              "moe_permute: NULL output with max_rows > 0");
  return MOE_OK;
}

moe_status permute_impl(int64_t T, int64_t h, int64_t E, int64_t K, int32_t dtype, const void* x,
                        const uint8_t* routing_map, const float* probs, int64_t max_rows,
                        void* permuted_x, float* permuted_probs, int32_t* sorted_token,
                        int32_t* row_id_map, int32_t* expert_offsets, void* workspace,
                        size_t workspace_bytes, hipStream_t s, const int32_t* given_blkoff,
                        const int32_t* given_totals) {
  const moe_status st = permute_check(T, h, E, K, dtype, x, routing_map, probs, max_rows,
                                      permuted_x, permuted_probs, sorted_token, row_id_map,
                                      expert_offsets);
  if (st != MOE_OK) return st;
  if (T == 0) {
    launch_fill_i32(expert_offsets, E + 1, 0, s);
    return check_launch("moe_permute(T=0)");
  }
  const int64_t nblk = ceil_div(T, kCountBlock);
  const int32_t* blkoff = given_blkoff;
  const int32_t* totals = given_totals;
  if (!blkoff) {
    const size_t need = moe_permute_workspace_size(T, E);
    MOE_REQUIRE(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE,
                "moe_permute: workspace of %zu bytes given, %zu needed", workspace_bytes, need);
    int32_t* hist = static_cast<int32_t*>(workspace);
    int32_t* off = hist + align_up(static_cast<size_t>(nblk * E) * sizeof(int32_t), 256) / 4;
    int32_t* tot = off + align_up(static_cast<size_t>(nblk * E) * sizeof(int32_t), 256) / 4;
    launch_block_hist(routing_map, T, E, hist, s);
    launch_count_scan(hist, nblk, E, -1, off, tot, s);
    blkoff = off;
    totals = tot;
  }
  const int esize = dtype == MOE_BF16 ? 2 : 4;
  const int chunks = static_cast<int>(h * esize / 16);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s,
                     routing_map, probs, static_cast<const uint4*>(x), T, static_cast<int>(E),
                     static_cast<int>(K), chunks, blkoff, totals, expert_offsets, max_rows,
                     static_cast<uint4*>(permuted_x), permuted_probs, sorted_token, row_id_map);
  return check_launch("moe_permute");
}

}  // namespace moe

extern "C" moe_status moe_permute(int64_t T, int64_t h, int64_t E, int64_t K, int32_t dtype,
                                  const void* x, const uint8_t* routing_map, const float* probs,
                                  int64_t max_rows, void* permuted_x, float* permuted_probs,
                                  int32_t* sorted_token, int32_t* row_id_map,
                                  int32_t* expert_offsets, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return permute_impl(T, h, E, K, dtype, x, routing_map, probs, max_rows, permuted_x,
                      permuted_probs, sorted_token, row_id_map, expert_offsets, workspace,
                      workspace_bytes, as_stream(stream), nullptr, nullptr);
}
