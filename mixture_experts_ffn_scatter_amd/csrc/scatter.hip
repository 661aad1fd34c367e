// moe_scatter_endpoints: grouped-layout scatter with int32 expert ends and
// fused per-32 FP8/UE8M0 quantisation of the routed token rows, on gfx950.
//
// The layout is the live-row layout of "Blackwell FP4 MoE: live-row
// boundary", section 2: start_e = align_up(end_{e-1}, A), end_e = start_e +
// count_e; the scatter writes the int32 ends itself, with no device-to-host
// read of the counts. Rows of one expert follow the flattened route order
// r = t*k+s, so the permutation is unique.
//
// Two launches, neither of which depends on a host-visible count. Tokens are
// grouped in blocks of TB (64, doubled while the block-by-expert count table
// would not fit in LDS). With a small table (<= 64 token blocks, <= 256
// local experts):
//   1. count - one block per token block: its routes counted per expert
//              with LDS atomics (counts need no order) into counts[w][e].
//   2. rows  - every block first redoes the small scan from the counts
//              (expert totals, the aligned exclusive scan over experts - the
//              endpoint recurrence - and its token block's offset inside
//              each expert; block 0 writes expert_ends), then one wave per
//              token: the rank of each local route is the number of earlier
//              routes of its token block with the same id (ballots over the
//              block's ids, read with the token's own ids), row = start_e +
//              block offset + rank; the x row is loaded after the ids,
//              quantised in registers and copied into every destination row
//              (codes coalesced 8 bytes per lane, packed scales assembled
//              across 16 lanes and stored MN-major).
// With a larger table, launch 1 is one block that counts every route and
// does the scans once (block offsets and starts in the workspace), and the
// rows kernel reads them instead of scanning.
#include "common.h"

#include <mutex>

namespace moe {

constexpr int kTokBlock = 64;       // smallest token block
constexpr int kScatterMaxE = 1024;
constexpr int kScatterMaxK = 32;
constexpr int kCountLds = 32768;    // (token block, expert) counters held in LDS

// token block size: 64, doubled until ceil(T / TB) * E_local counters fit
inline int scatter_token_block(int T, int E_local) {
  int tb = kTokBlock;
  while ((long long)((T + tb - 1) / tb) * E_local > kCountLds) tb *= 2;
  return tb;
}

// Block-wide exclusive scan of one int per thread (1024 threads).
__device__ int block_exclusive_scan_1024(int v, int* wave_tot) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_tot[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    int x = lane < 16 ? wave_tot[lane] : 0;
    int ix = x;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int o = __shfl_up(ix, d, 64);
      if (lane >= d) ix += o;
    }
    if (lane < 16) wave_tot[16 + lane] = ix - x;  // exclusive wave offsets
  }
  __syncthreads();
  return wave_tot[16 + wid] + incl - v;
}

constexpr int kCountBatch = 32;     // ids in flight per lane

// slab > 0: the masked slab layout (starts e * slab, and expert_ends receives
// masked_m = min(count, slab))
__global__ __launch_bounds__(1024) void scatter_count_scan_kernel(
    const int32_t* __restrict__ ids, int T, int k, int expert_start, int E_local, int A, int slab,
    int TB, int W, int32_t* __restrict__ offsets, int32_t* __restrict__ starts,
    int32_t* __restrict__ expert_ends) {
  __shared__ int s_cnt[kCountLds];
  __shared__ int s_tot[kScatterMaxE];
  __shared__ int wave_tot[32];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = T * k;
  const int rpb = TB * k;                // routes per token block
  // wave wid counts token blocks wid, wid+16, ...: a flat list of 64-route
  // chunks (block j of the wave, chunk c of the block) walked with
  // wave-uniform counters, so no route needs a division
  const int cpb = (rpb + 63) / 64;       // chunks per block
  const int nq = ((W - wid + 15) / 16) * cpb;
  int id[kCountBatch];
  int blk[kCountBatch];
  int qj = 0, qc = 0;                    // position of the next chunk to load
  auto load = [&](int q0) {
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) {
      const int b = wid + 16 * qj;
      const int o = qc * 64 + lane;
      const int r = b * rpb + o;
      // unpredicated, in-bounds load; validity goes in blk (-1: no route)
      id[u] = ids[min(r, n - 1)];
      blk[u] = (q0 + u < nq && o < rpb && r < n) ? b : -1;
      if (++qc == cpb) {
        qc = 0;
        ++qj;
      }
    }
  };
  if (nq > 0) load(0);                   // in flight while the counters are cleared
  for (int i = tid; i < W * E_local; i += 1024) s_cnt[i] = 0;
  __syncthreads();
  for (int q0 = 0; q0 < nq; q0 += kCountBatch) {
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) {
      const int e = id[u] - expert_start;
      if (blk[u] >= 0 && e >= 0 && e < E_local) atomicAdd(&s_cnt[blk[u] * E_local + e], 1);
    }
    if (q0 + kCountBatch < nq) load(q0 + kCountBatch);
  }
  __syncthreads();
  // per expert: exclusive scan over the token blocks, 64 blocks at a time
  for (int e = wid; e < E_local; e += 16) {
    int carry = 0;
    for (int w0 = 0; w0 < W; w0 += 64) {
      const int w = w0 + lane;
      const int c = w < W ? s_cnt[w * E_local + e] : 0;
      int incl = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
      }
      if (w < W) offsets[(size_t)w * E_local + e] = carry + incl - c;
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) s_tot[e] = carry;
  }
  __syncthreads();
  const int e = tid;
  const int total = e < E_local ? s_tot[e] : 0;
  const int aligned = e < E_local ? align_up_dev(total, A) : 0;
  const int start = block_exclusive_scan_1024(aligned, wave_tot);
  if (e < E_local) {
    starts[e] = slab > 0 ? e * slab : start;
    expert_ends[e] = slab > 0 ? min(total, slab) : start + total;
  }
}

// One block per token block: its routes counted per expert with LDS
// atomics, written to counts[w][e]. Used when the rows kernel scans the
// counts itself.
constexpr int kCntBatch = 4;        // ids in flight per thread

__global__ __launch_bounds__(256) void scatter_count_kernel(const int32_t* __restrict__ ids,
                                                            int n, int expert_start, int E_local,
                                                            int rpb,
                                                            int32_t* __restrict__ counts) {
  __shared__ int s[kScatterMaxE];
  const int w = blockIdx.x;
  const int tid = threadIdx.x;
  const int rb = w * rpb;
  const int re = min(n, rb + rpb);
  int id[kCntBatch];
  auto load = [&](int r0) {
#pragma unroll
    for (int u = 0; u < kCntBatch; ++u) id[u] = ids[min(r0 + u * 256 + tid, n - 1)];
  };
  load(rb);                           // in flight while the counters are cleared
  for (int e = tid; e < E_local; e += 256) s[e] = 0;
  __syncthreads();
  for (int r0 = rb; r0 < re; r0 += 256 * kCntBatch) {
#pragma unroll
    for (int u = 0; u < kCntBatch; ++u) {
      const int e = id[u] - expert_start;
      if (r0 + u * 256 + tid < re && e >= 0 && e < E_local) atomicAdd(&s[e], 1);
    }
    if (r0 + 256 * kCntBatch < re) load(r0 + 256 * kCntBatch);
  }
  __syncthreads();
  for (int e = tid; e < E_local; e += 256) counts[(size_t)w * E_local + e] = s[e];
}

constexpr int kRowsWaves = 4;    // tokens per block
constexpr int kRowsBatch = 8;    // 512-column chunks held in registers at once
constexpr int kPrevBatch = 8;    // 64-route chunks of earlier ids loaded at once

constexpr int kScanMaxW = 64;    // rows-kernel scan: token blocks
constexpr int kScanMaxE = 256;   // rows-kernel scan: local experts

// SCAN: `meta` holds the per-(token block, expert) counts and every block
// redoes the small scan itself (start_e plus the token block's offset inside
// expert e, for all e; block 0 also writes expert_ends). Otherwise `meta`
// holds the block offsets and `starts` the expert starts.
// G128: one UE8M0 byte per 128 columns instead of per 32, packed four to a
// word over 512 columns ([ceil(H/512)][M_cap] words; bytes of groups past H
// are 0).
// SLAB: the masked slab layout ("DeepGEMM FusedMoE on Blackwell (sglang)",
// section 2.2.4): expert e's rows start at e * slab, a route whose rank in
// its expert reaches slab is not placed (row -1), expert_ends receives
// masked_m = min(count, slab), M_cap = E_local * slab, and the scale words
// are MN-major per expert ([e][word][row - e slab]).
template <bool SCAN, bool G128, bool SLAB>
__global__ __launch_bounds__(64 * kRowsWaves) void scatter_rows_kernel(
    const int32_t* __restrict__ ids, int T, int k, int expert_start, int E_local, int A,
    int M_cap, int slab, int TB, int W, const uint16_t* __restrict__ x, int H,
    const int32_t* __restrict__ meta, const int32_t* __restrict__ starts,
    int32_t* __restrict__ expert_ends, int32_t* __restrict__ route_row,
    uint8_t* __restrict__ xq, int32_t* __restrict__ xs) {
  __shared__ int s_base[SCAN ? kScanMaxE : 1];
  __shared__ int s_wsum[kRowsWaves];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = blockIdx.x * kRowsWaves + wid;
  const bool tok = t < T;                // wave-uniform
  const int wblk = blockIdx.x * kRowsWaves / TB;   // TB % kRowsWaves == 0: one token block
  const int rt = t * k;                  // the token's first route
  const int rb = wblk * TB * k;          // its token block's first route
  const int nprev = rt - rb;             // earlier routes of the block
  // an id no local route has, for lanes past the earlier routes
  const int none = expert_start > INT_MIN ? expert_start - 1 : INT_MAX;
  // level 1: the token's ids (lanes < k) and the block's earlier ids, together
  int id = none;
  if (tok && lane < k) id = ids[rt + lane];
  int prev[kPrevBatch];
  auto load_prev = [&](int c0) {
#pragma unroll
    for (int u = 0; u < kPrevBatch; ++u) {
      const int j = c0 + u * 64 + lane;
      prev[u] = (tok && j < nprev) ? ids[rb + j] : none;
    }
  };
  load_prev(0);
  if constexpr (SCAN) {
    // thread e: expert e's total and its count in earlier token blocks; then
    // the aligned exclusive scan over experts across the block's threads
    const int e = threadIdx.x;
    int total = 0, before = 0;
    if (e < E_local) {
      int c[kScanMaxW];
#pragma unroll
      for (int w = 0; w < kScanMaxW; ++w) c[w] = meta[(size_t)min(w, W - 1) * E_local + e];
#pragma unroll
      for (int w = 0; w < kScanMaxW; ++w) {
        const int v = w < W ? c[w] : 0;
        total += v;
        before += w < wblk ? v : 0;
      }
    }
    const int aligned = e < E_local ? align_up_dev(total, A) : 0;
    int incl = aligned;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    if (lane == 63) s_wsum[wid] = incl;
    __syncthreads();
    int start = incl - aligned;
    for (int v = 0; v < wid; ++v) start += s_wsum[v];
    if (e < E_local) {
      if constexpr (SLAB) {
        s_base[e] = e * slab + before;
        if (blockIdx.x == 0) expert_ends[e] = min(total, slab);
      } else {
        s_base[e] = start + before;
        if (blockIdx.x == 0) expert_ends[e] = start + total;
      }
    }
    __syncthreads();
  }
  if (!tok) return;
  const int ev = id - expert_start;
  const bool local = lane < k && id != none && ev >= 0 && ev < E_local;
  const uint64_t lmask = __ballot(local);
  if (lmask == 0ull) {                   // wave-uniform: no local route
    if (lane < k) route_row[rt + lane] = -1;
    return;
  }
  // rank of each local slot: earlier slots of the token, then earlier
  // routes of the block, with the same id (lane s keeps slot s's rank).
  // Done before the next loads are issued: a loop with loads in it would
  // make every load in flight complete before it.
  int rank = 0;
  for (uint64_t m = lmask; m; m &= m - 1) {
    const int s = __ffsll((unsigned long long)m) - 1;
    const int key = __builtin_amdgcn_readlane(id, s);
    const int c = __popcll(__ballot(lane < s && id == key));
    if (lane == s) rank = c;
  }
  for (int c0 = 0;;) {
    for (uint64_t m = lmask; m; m &= m - 1) {
      const int s = __ffsll((unsigned long long)m) - 1;
      const int key = __builtin_amdgcn_readlane(id, s);
      int c = 0;
#pragma unroll
      for (int u = 0; u < kPrevBatch; ++u) c += __popcll(__ballot(prev[u] == key));
      if (lane == s) rank += c;
    }
    c0 += 64 * kPrevBatch;
    if (c0 >= nprev) break;              // wave-uniform
    load_prev(c0);
  }
  // level 2: start and block offset of the local slots' experts, and the x row
  const int ec = local ? ev : 0;         // unpredicated: every lane reads a valid entry
  int base;
  if constexpr (SCAN) {
    base = s_base[ec];
  } else {
    base = starts[ec] + meta[(size_t)wblk * E_local + ec];
  }
  const uint16_t* xr = x + (size_t)t * H;
  const int nch = (H + 511) / 512;
  uint4 raw[kRowsBatch];
  // unpredicated loads (columns past H read the row's last 8 and are not
  // used), so that each chunk waits only for its own load
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int j = 0; j < kRowsBatch; ++j) {
      const int col = min((c0 + j) * 512 + lane * 8, H - 8);
      raw[j] = *reinterpret_cast<const uint4*>(xr + col);
    }
  };
  load_batch(0);
  int row = -1;
  if (local) {
    row = base + rank;
    if constexpr (SLAB) {
      if (row - ev * slab >= slab) row = -1;   // the expert's slab is full: not placed
    }
    if (row >= M_cap) row = -1;           // corrupt metadata: never write past the buffer
  }
  const uint64_t live = __ballot(row >= 0);
  if (lane < k) route_row[rt + lane] = row;

  for (int c0 = 0; c0 < nch; c0 += kRowsBatch) {
    if (c0 > 0) load_batch(c0);
    // chunk by chunk: the stores of one chunk overlap the next chunk's math
#pragma unroll
    for (int j = 0; j < kRowsBatch; ++j) {
      const int col = (c0 + j) * 512 + lane * 8;
      if ((c0 + j) * 512 >= H) break;     // wave-uniform
      const float v[8] = {bf16_lo(raw[j].x), bf16_hi(raw[j].x), bf16_lo(raw[j].y),
                          bf16_hi(raw[j].y), bf16_lo(raw[j].z), bf16_hi(raw[j].z),
                          bf16_lo(raw[j].w), bf16_hi(raw[j].w)};
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      if constexpr (G128) {               // the 128-column group: 16 lanes
        amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 8, 64));
      }
      const uint32_t b = ue8m0_byte_of_amax(amax);
      const float inv = e8m0_reciprocal(b);
      uint32_t lo = 0, hi = 0;
      lo = cvt_e4m3x2<false>(v[0] * inv, v[1] * inv, lo);
      lo = cvt_e4m3x2<true>(v[2] * inv, v[3] * inv, lo);
      hi = cvt_e4m3x2<false>(v[4] * inv, v[5] * inv, hi);
      hi = cvt_e4m3x2<true>(v[6] * inv, v[7] * inv, hi);
      uint32_t wd;
      if constexpr (G128) {
        // byte q of the chunk's word: the group of lanes 16q .. 16q + 15
        const bool in = (c0 + j) * 512 + 128 * (lane >> 4) < H;
        wd = (in ? b : 0u) << (8 * (lane >> 4));
        wd |= __shfl_xor(wd, 16, 64);
        wd |= __shfl_xor(wd, 32, 64);
      } else {
        wd = b << (8 * ((lane >> 2) & 3));
        wd |= __shfl_xor(wd, 4, 64);
        wd |= __shfl_xor(wd, 8, 64);
      }
      for (uint64_t m = live; m; m &= m - 1) {   // wave-uniform loop over destination rows
        const int s = __ffsll((unsigned long long)m) - 1;
        const int r = __builtin_amdgcn_readlane(row, s);
        // scale word w of row r: [w][r] over the whole buffer, or
        // [e][w][r - e slab] inside expert e's slab
        size_t xs0 = r;
        int xss = M_cap;
        if constexpr (SLAB) {
          const int WN = G128 ? (H + 511) >> 9 : H >> 7;
          xs0 = (size_t)__builtin_amdgcn_readlane(ev, s) * (size_t)(WN - 1) * (size_t)slab + r;
          xss = slab;
        }
        if (col < H) {
          *reinterpret_cast<uint2*>(xq + (size_t)r * H + col) = make_uint2(lo, hi);
          if constexpr (G128) {
            if (lane == 0) xs[xs0 + (size_t)(c0 + j) * xss] = (int32_t)wd;
          } else {
            if ((lane & 15) == 0) xs[xs0 + (size_t)(col >> 7) * xss] = (int32_t)wd;
          }
        }
      }
    }
  }
}

// Plain fill used for the degenerate cases (a kernel, not a memset node, so
// that graph capture of the call stays safe).
__global__ void fill_i32_kernel(int32_t* __restrict__ p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

static int fill_i32(int32_t* p, int n, int32_t v, hipStream_t st) {
  if (n <= 0) return MOE_OK;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

}  // namespace moe

extern "C" size_t moe_scatter_workspace_bytes(int T, int k, int E_local) {
  (void)k;
  if (T <= 0 || E_local <= 0) return 0;
  const int tb = moe::scatter_token_block(T, E_local);
  const size_t W = (size_t)(T + tb - 1) / tb;
  return (W + 1) * (size_t)E_local * sizeof(int32_t);   // block offsets, then starts
}

namespace moe {
// Host-side checks of the scatter's sizes and pointers (no side effects).
// slab > 0 (the masked slab layout): M_cap = E_local * slab, and any slab
// size is valid (routes past a full slab are not placed).
static int scatter_validate(const int32_t* topk_ids, int T, int k, int E_local, int A, int M_cap,
                            const uint16_t* x, int H, int32_t* expert_ends, int32_t* route_row,
                            uint8_t* xq, int32_t* xs, int slab = 0) {
  if (T < 0 || k < 1 || k > kScatterMaxK || E_local < 0 || E_local > kScatterMaxE || A < 1 ||
      M_cap < 0 || H <= 0 || (long long)T * k > INT_MAX)
    return MOE_ERR_SHAPE;
  if (H % 128 != 0 || M_cap % 4 != 0) return MOE_ERR_ALIGN;
  if (slab == 0 && (long long)M_cap < (long long)T * k + (long long)E_local * A)
    return MOE_ERR_CAPACITY;
  if (E_local == 0 && T == 0) return MOE_OK;
  if (!expert_ends && E_local > 0) return MOE_ERR_NULL;
  if (T > 0 && (!topk_ids || !x || !route_row || !xq || !xs)) return MOE_ERR_NULL;
  return MOE_OK;
}

static int scatter_endpoints(const int32_t* topk_ids, int T, int k, int expert_start, int E_local,
                             int A, int M_cap, const uint16_t* x, int H, int32_t* expert_ends,
                             int32_t* route_row, uint8_t* xq, int32_t* xs, void* workspace,
                             size_t workspace_bytes, void* stream, bool g128, int slab = 0) {
  const int bad = scatter_validate(topk_ids, T, k, E_local, A, M_cap, x, H, expert_ends, route_row,
                                   xq, xs, slab);
  if (bad != MOE_OK) return bad;
  if (E_local == 0 && T == 0) return MOE_OK;
  if (T == 0) {
    // no routes: every expert is empty, ends are all zero
    return fill_i32(expert_ends, E_local, 0, (hipStream_t)stream);
  }
  if (E_local == 0) return fill_i32(route_row, T * k, -1, (hipStream_t)stream);
  const size_t need = moe_scatter_workspace_bytes(T, k, E_local);
  if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int TB = scatter_token_block(T, E_local);
  const int W = (T + TB - 1) / TB;
  int32_t* meta = (int32_t*)workspace;   // counts or block offsets [W][E_local]
  int32_t* starts = meta + (size_t)W * E_local;
  const dim3 rows_grid((T + kRowsWaves - 1) / kRowsWaves);
  if (W <= kScanMaxW && E_local <= kScanMaxE) {
    // small count table: per-block counts, and each rows block scans them
    hipLaunchKernelGGL(scatter_count_kernel, dim3(W), dim3(256), 0, st, topk_ids, T * k,
                       expert_start, E_local, TB * k, meta);
    MOE_CHECK_LAUNCH();
    auto rows_kernel = slab > 0 ? scatter_rows_kernel<true, false, true>
                       : g128 ? scatter_rows_kernel<true, true, false>
                              : scatter_rows_kernel<true, false, false>;
    hipLaunchKernelGGL(rows_kernel, rows_grid, dim3(64 * kRowsWaves), 0, st, topk_ids, T, k, expert_start,
                       E_local, A, M_cap, slab, TB, W, x, H, meta, starts, expert_ends, route_row,
                       xq, xs);
    MOE_CHECK_LAUNCH();
  } else {
    hipLaunchKernelGGL(scatter_count_scan_kernel, dim3(1), dim3(1024), 0, st, topk_ids, T, k,
                       expert_start, E_local, A, slab, TB, W, meta, starts, expert_ends);
    MOE_CHECK_LAUNCH();
    auto rows_kernel = slab > 0 ? scatter_rows_kernel<false, false, true>
                       : g128 ? scatter_rows_kernel<false, true, false>
                              : scatter_rows_kernel<false, false, false>;
    hipLaunchKernelGGL(rows_kernel, rows_grid, dim3(64 * kRowsWaves), 0, st, topk_ids, T, k, expert_start,
                       E_local, A, M_cap, slab, TB, W, x, H, meta, starts, expert_ends, route_row,
                       xq, xs);
    MOE_CHECK_LAUNCH();
  }
  return MOE_OK;
}
}  // namespace moe

extern "C" int moe_scatter_endpoints(const int32_t* topk_ids, int T, int k, int expert_start,
                                     int E_local, int A, int M_cap, const uint16_t* x, int H,
                                     int32_t* expert_ends, int32_t* route_row, uint8_t* xq,
                                     int32_t* xs, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  return moe::scatter_endpoints(topk_ids, T, k, expert_start, E_local, A, M_cap, x, H, expert_ends,
                                route_row, xq, xs, workspace, workspace_bytes, stream, false);
}

namespace moe {
// Device scratch of moe_scatter_endpoints_noalloc, in place of the caller's
// workspace. The largest workspace a valid call needs is the counter table
// (at most kCountLds (token block, expert) entries: scatter_token_block grows
// the block until they fit) plus one start per expert.
constexpr size_t kScatterScratchBytes = (size_t)(kCountLds + kScatterMaxE) * sizeof(int32_t);
static __device__ __align__(256) uint8_t scratch[kScatterScratchBytes];

// The array's address on each device, looked up once per device (each GPU
// holds its own copy at its own address). Host code uses these addresses,
// never the symbol itself.
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace moe

extern "C" int moe_scatter_endpoints_noalloc(const int32_t* topk_ids, int T, int k,
                                             int expert_start, int E_local, int A, int M_cap,
                                             const uint16_t* x, int H, int32_t* expert_ends,
                                             int32_t* route_row, uint8_t* xq, int32_t* xs,
                                             void* stream) {
  // the argument checks, then the scratch size, before anything else
  const int bad = moe::scatter_validate(topk_ids, T, k, E_local, A, M_cap, x, H, expert_ends,
                                        route_row, xq, xs);
  if (bad != MOE_OK) return bad;
  if (T > 0 && E_local > 0 && moe_scatter_workspace_bytes(T, k, E_local) > moe::kScatterScratchBytes)
    return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  if (T > 0 && E_local > 0) {
    const int st = moe::scratch_on_current_device(&ws);
    if (st != MOE_OK) return st;
  }
  // the counters and offsets in the scratch are written in full before they
  // are read, so nothing carried over from an earlier call is ever used
  return moe::scatter_endpoints(topk_ids, T, k, expert_start, E_local, A, M_cap, x, H, expert_ends,
                                route_row, xq, xs, ws, moe::kScatterScratchBytes, stream, false);
}

extern "C" int moe_scatter_endpoints_g128(const int32_t* topk_ids, int T, int k, int expert_start,
                                          int E_local, int A, int M_cap, const uint16_t* x, int H,
                                          int32_t* expert_ends, int32_t* route_row, uint8_t* xq,
                                          int32_t* xs, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  return moe::scatter_endpoints(topk_ids, T, k, expert_start, E_local, A, M_cap, x, H, expert_ends,
                                route_row, xq, xs, workspace, workspace_bytes, stream, true);
}

extern "C" int moe_scatter_masked(const int32_t* topk_ids, int T, int k, int expert_start,
                                  int E_local, int m_pad, const uint16_t* x, int H,
                                  int32_t* masked_m, int32_t* route_row, uint8_t* xq, int32_t* xs,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (E_local < 0 || m_pad < 0) return MOE_ERR_SHAPE;
  if (m_pad % 4 != 0) return MOE_ERR_ALIGN;
  if ((long long)E_local * m_pad >= (1LL << 31)) return MOE_ERR_SHAPE;
  if (E_local > 0 && m_pad == 0) return MOE_ERR_SHAPE;
  return moe::scatter_endpoints(topk_ids, T, k, expert_start, E_local, 1, E_local * m_pad, x, H,
                                masked_m, route_row, xq, xs, workspace, workspace_bytes, stream,
                                false, m_pad);
}
