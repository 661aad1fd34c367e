// moe_grouped_gemm1 / moe_grouped_gemm2: grouped MX GEMMs over the live rows
// of the aligned expert layout, on gfx950 scaled MFMA; and
// moe_pack_mx_weights, the load-time weight preparation they consume.
//
//   out[m, n] = sum_k X[m, k] * W_e[n, k]      for m in [start_e, end_e)
//
// X is E4M3 with one UE8M0 byte per 32 columns (packed MN-major, four per
// int32), W_e is E2M1 with one E8M0 byte per 32 columns ("Blackwell DeepGEMM
// FusedMoE (sglang)", sections 2.3 / 2.5 / 3.3 and 3.8: contiguous grouped
// FP8 x FP4 GEMM with (1,32) weight scales; here the activation recipe is
// (1,32) as well). "Blackwell FP4 MoE: live-row boundary", section 2: both
// GEMMs take the int32 expert ends; rows outside [start_e, end_e) are
// neither read nor written.
//
// Mapping onto V_MFMA_SCALE_F32_16X16X128_F8F6F4 (lane layout measured on
// gfx950 with a one-instruction probe): the weight tile is the A operand
// (16 output columns x 128 k, E2M1, 16 bytes per lane) and the activation
// tile the B operand (128 k x 16 rows, E4M3, 32 bytes per lane). With
// g = lane/16, an E2M1 operand holds k-slice [32g, 32g+32) of row lane%16 in
// order (low nibble first), while an E4M3 operand holds k [16g, 16g+16) in
// its first four dwords and k [64+16g, 64+16g+16) in the last four. The
// E8M0 scale of row r and 32-wide k-block b is read from lane r + 16b. The
// 16x16 fp32 result gives lane l four consecutive output columns of row
// l%16, stored as one 8-byte bf16 write.
//
// Weight preparation (once, at load time; "Blackwell DeepGEMM FusedMoE
// (sglang)", section 2.1: weights are rearranged into the layout the GEMM
// consumes, so that the run-time GEMM never touches the checkpoint layout):
// codes are stored in MFMA fragment order, one contiguous 1 KB chunk per
// (16-column block, 128-wide k-step), and scales as one 8-byte word per lane
// per (16-column block, 8 k-steps). A wave then streams its weights with
// fully coalesced 16-byte loads straight into registers.
//
// Work decomposition. An item is (n-tile of 256 columns, expert, m-chunk of
// up to 128 live rows). Items are listed n-tile-major and the list is cut
// into 8 equal contiguous ranges, one per XCD (block b runs on XCD b % 8);
// the blocks of an XCD take its items round-robin, so the m-chunks of one
// (expert, n-tile) run side by side on one XCD and share its weight slice
// in that L2, and every XCD streams about 1/8 of the weights. The list is
// rebuilt inside every block from expert_ends (a block-wide scan), so the
// grid depends only on host-known sizes and no count is read back.
//
// Inside an item, the 8 waves form 2 row groups x 4 column groups: wave
// (rg, cg) computes rows [64rg, 64rg+64) x columns [64cg, 64cg+64) of the
// tile, so an activation fragment read from LDS feeds 4 MFMAs. Its weight
// fragments go global -> registers 4 k-steps ahead (both row groups read
// the same fragments, the second from cache; a row group with no live rows
// reads nothing). The activation chunk (shared by all waves) is loaded
// 3 k-steps ahead into registers, one 16-row block per wave, and written
// to a two-slot LDS ring one step ahead; one barrier per k-step. Loads use buffer resources whose
// range ends at the last live row (or column): lanes past it read zeros
// without touching memory, so padding rows are never read and every wave
// issues the same instruction stream.
#include "common.h"

#ifndef GEMM_CB
#define GEMM_CB 2
#endif
#ifndef GEMM_WD
#define GEMM_WD 4
#endif
#ifndef GEMM_XD
#define GEMM_XD 2
#endif

namespace moe {

constexpr int kGemmThreads = 512;  // 8 waves
constexpr int kGemmBM = 128;       // rows per item (8 blocks of 16)
constexpr int kGemmBN = 256;       // columns per item (16 blocks of 16)
constexpr int kGemmCB = GEMM_CB;                        // column blocks per wave
constexpr int kGemmNCG = kGemmBN / 16 / kGemmCB;            // column groups
constexpr int kGemmMB = (kGemmBM / 16) / (kGemmThreads / 64 / kGemmNCG);  // row blocks per wave
static_assert(kGemmNCG * (kGemmBM / 16 / kGemmMB) == kGemmThreads / 64, "wave grid");
constexpr int kGemmU = 8;          // k-loop unroll (one weight-scale word group)
constexpr int kGemmWD = GEMM_WD;   // weight prefetch distance in k-steps
constexpr int kGemmXD = GEMM_XD;   // activation register prefetch depth
constexpr int kGemmMaxE = 1024;
constexpr uint32_t kOob = 0x80000000u;  // buffer offset past any range: reads zero, no traffic

// One LDS slot: the activation chunk of one k-step in MFMA fragment order
// (x[mb][h][lane] = 16 bytes of row 16mb + lane%16, k [64h + 16(lane/16), +16))
// and its 128 packed scale words.
struct __attribute__((aligned(16))) GemmXSlot {
  uint8_t x[kGemmBM / 16][2][64 * 16];
  uint32_t xs[kGemmBM];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // raw buffer (stride 0); word 3 as for every gfx9 raw buffer
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// Workgroup barrier without the release fence of __syncthreads() (which
// would wait for every outstanding global load and empty the prefetch):
// this wave's LDS writes are completed first, which is all the ring needs.
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ int block_exclusive_scan(int v, int* tmp) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) tmp[wid] = incl;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wid; ++w) off += tmp[w];
  __syncthreads();
  return off + incl - v;
}

// One work item's load parameters. Buffer ranges end at the item's last
// live column block (weights) and last live row (activations); an absent
// item has empty ranges, so every load from it reads zero without touching
// memory.
struct GemmItem {
  __amdgpu_buffer_rsrc_t wr, sr, xr, xsr;
  uint32_t wo[kGemmCB], so[kGemmCB];   // per-lane weight / scale offsets
  uint32_t xso;                        // per-lane scale-word offset (row part)
  int r0, rows, nblk, mlive, cb0, ncb, valid;
};

__global__ __launch_bounds__(kGemmThreads, 1) void grouped_mx_gemm_kernel(
    const uint8_t* __restrict__ X, const int32_t* __restrict__ Xs,
    const int32_t* __restrict__ expert_ends, int E_local, int A, int M_cap, int K, int N,
    const uint8_t* __restrict__ Wp, const uint8_t* __restrict__ Sp, uint16_t* __restrict__ out) {
  __shared__ GemmXSlot xl[2];
  __shared__ int s_prefix[kGemmMaxE + 1];
  __shared__ int s_tmp[kGemmThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int rg = wid / kGemmNCG;         // row group: row blocks [MB*rg, MB*rg+MB)
  const int cg = wid % kGemmNCG;         // column group: column blocks [CB*cg, CB*cg+CB)
  const int KS = K / 128;                // k-steps
  const int KS8 = (KS + 7) / 8;          // 8-step scale groups
  const int NB = N / 16;                 // column blocks
  const int NT = (N + kGemmBN - 1) / kGemmBN;
  // With KS a multiple of the weight prefetch distance (K % 512 == 0) the
  // register rings line up across items, and the loads of the next item's
  // first steps are issued during the current item's last ones. Otherwise
  // each item starts with its own prologue.
  const bool chain = KS % kGemmWD == 0;

  // m-chunks per expert and their exclusive scan (2 experts per thread)
  int cnt[2];
  int local_sum = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = tid * 2 + j;
    cnt[j] = 0;
    if (e < E_local) {
      int s, en;
      expert_range(expert_ends, e, A, M_cap, s, en);
      cnt[j] = (en - s + kGemmBM - 1) / kGemmBM;
    }
    local_sum += cnt[j];
  }
  int run = block_exclusive_scan(local_sum, s_tmp);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = tid * 2 + j;
    if (e < E_local) s_prefix[e] = run;
    run += cnt[j];
  }
  if (tid == kGemmThreads - 1) s_prefix[E_local] = run;
  __syncthreads();
  const int MT = s_prefix[E_local];      // m-chunks over all experts
  const int L = MT * NT;                 // items

  // this block's XCD range of the item list and its slot in it
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int nslot = gridDim.x >> 3;      // the grid is a multiple of 8
  const int i_end = (int)(((long long)L * (xcd + 1)) / 8);
  const int first = (int)(((long long)L * xcd) / 8) + slot;

  const uint32_t xo = (uint32_t)(16 * wid + l16) * (uint32_t)K + 16 * g;   // staged row block wid

  auto make_item = [&](int item) {
    GemmItem it;
    it.valid = item < i_end;
    if (!it.valid) {
      it.wr = it.sr = it.xr = it.xsr = make_rsrc(Wp, 0u);
#pragma unroll
      for (int c = 0; c < kGemmCB; ++c) it.wo[c] = it.so[c] = kOob;
      it.xso = kOob;
      it.r0 = it.rows = it.nblk = it.mlive = it.cb0 = it.ncb = 0;
      return it;
    }
    const int nt = item / MT;
    const int j = item - nt * MT;
    int lo = 0, hi = E_local - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_prefix[mid] <= j) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    int start, end;
    expert_range(expert_ends, e, A, M_cap, start, end);
    it.r0 = start + (j - s_prefix[e]) * kGemmBM;
    it.rows = min(kGemmBM, end - it.r0);                  // >= 1
    it.nblk = (it.rows + 15) >> 4;
    it.mlive = min(max(it.nblk - kGemmMB * rg, 0), kGemmMB);
    it.cb0 = nt * (kGemmBN / 16);
    it.ncb = min(kGemmBN / 16, NB - it.cb0);
    it.wr = make_rsrc(Wp + ((size_t)e * NB + it.cb0) * KS * 1024, (uint32_t)(it.ncb * KS) * 1024u);
    it.sr = make_rsrc(Sp + ((size_t)e * NB + it.cb0) * KS8 * 512, (uint32_t)(it.ncb * KS8) * 512u);
    it.xr = make_rsrc(X + (size_t)it.r0 * K, (uint32_t)it.rows * (uint32_t)K);
    it.xsr = make_rsrc(Xs + it.r0, (uint32_t)((KS - 1) * M_cap + it.rows) * 4u);
#pragma unroll
    for (int c = 0; c < kGemmCB; ++c) {
      const int cb = kGemmCB * cg + c;
      const bool live = cb < it.ncb && it.mlive > 0;
      it.wo[c] = live ? (uint32_t)(cb * KS) * 1024u + lane * 16 : kOob;
      it.so[c] = live ? (uint32_t)(cb * KS8) * 512u + lane * 8 : kOob;
    }
    it.xso = (lane < 16 && 16 * wid + l16 < it.rows) ? (uint32_t)(16 * wid + l16) * 4u : kOob;
    return it;
  };

  // loads of step ks of item p (ks < KS)
  auto load_w = [&](const GemmItem& p, int ks, v4i* dst) {
#pragma unroll
    for (int c = 0; c < kGemmCB; ++c)
      dst[c] = __builtin_amdgcn_raw_buffer_load_b128(p.wr, p.wo[c] + ks * 1024, 0, 0);
  };
  auto load_s = [&](const GemmItem& p, int q, v2i* dst) {
#pragma unroll
    for (int c = 0; c < kGemmCB; ++c)
      dst[c] = __builtin_amdgcn_raw_buffer_load_b64(p.sr, p.so[c] + q * 512, 0, 0);
  };
  auto load_x = [&](const GemmItem& p, int ks, v4i* dst, uint32_t& ws) {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b128(p.xr, xo + ks * 128, 0, 0);
    dst[1] = __builtin_amdgcn_raw_buffer_load_b128(p.xr, xo + ks * 128 + 64, 0, 0);
    ws = __builtin_amdgcn_raw_buffer_load_b32(
        p.xsr, p.xso == kOob ? kOob : p.xso + (uint32_t)(ks * M_cap) * 4u, 0, 0);
  };
  auto store_x = [&](int sl, const v4i* src, uint32_t ws) {
    *reinterpret_cast<v4i*>(&xl[sl].x[wid][0][lane * 16]) = src[0];
    *reinterpret_cast<v4i*>(&xl[sl].x[wid][1][lane * 16]) = src[1];
    if (lane < 16) xl[sl].xs[16 * wid + lane] = ws;
  };

  v4i wbuf[kGemmWD][kGemmCB];
  v2i s_cur[kGemmCB], s_nxt[kGemmCB];
  v4i xbuf[kGemmXD][2];
  uint32_t xsb[kGemmXD];
  const GemmItem none = make_item(i_end);

  // prologue of an item: weights of steps 0..WD-1, scale groups 0 and 1,
  // activations of steps 0..XD-1 (step 0 goes to LDS slot 0 and its
  // registers take step XD); loads past the item read nothing
  auto prologue = [&](const GemmItem& p) {
#pragma unroll
    for (int s = 0; s < kGemmWD; ++s) load_w(s < KS ? p : none, s < KS ? s : 0, wbuf[s]);
    load_s(p, 0, s_cur);
    load_s(KS8 > 1 ? p : none, 1, s_nxt);
#pragma unroll
    for (int s = 0; s < kGemmXD; ++s) load_x(s < KS ? p : none, s < KS ? s : 0, xbuf[s], xsb[s]);
    store_x(0, xbuf[0], xsb[0]);
    load_x(kGemmXD < KS ? p : none, kGemmXD < KS ? kGemmXD : 0, xbuf[0], xsb[0]);
    ring_barrier();
  };

  int item = first;
  GemmItem cur = make_item(item);
  if (cur.valid) prologue(cur);
  while (cur.valid) {
    const GemmItem nxt = make_item(item + nslot);
    // loads for steps past the end of this item come from the next one
    const GemmItem& pf = chain ? nxt : none;

    v4f acc[kGemmCB][kGemmMB];
#pragma unroll
    for (int c = 0; c < kGemmCB; ++c)
#pragma unroll
      for (int i = 0; i < kGemmMB; ++i) acc[c][i] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int kb = 0; kb < KS; kb += kGemmU) {
      if (kb > 0) {
#pragma unroll
        for (int c = 0; c < kGemmCB; ++c) s_cur[c] = s_nxt[c];
      }
      // the scale group after the current one: this item's, else the next
      // item's group 0 (groups 0 and 1 of the first item come from the prologue)
      if (kb > 0) {
        const int q = kb / kGemmU + 1;
        load_s(q < KS8 ? cur : pf, q < KS8 ? q : 0, s_nxt);
      }
#pragma unroll
      for (int jj = 0; jj < kGemmU; ++jj) {
        const int ks = kb + jj;
        if (ks >= KS) break;
        // stage step ks+1 (of this item, else step 0 of the next) into the
        // other slot, then refill its registers (xbuf[i % XD] holds step i)
        const int xi = (jj + 1) % kGemmXD;
        if (ks + 1 < KS || chain) store_x((jj + 1) & 1, xbuf[xi], xsb[xi]);
        {
          const int t = ks + 1 + kGemmXD;
          load_x(t < KS ? cur : pf, t < KS ? t : t - KS, xbuf[xi], xsb[xi]);
        }

        // compute step ks from slot ks % 2 (kb and KS are even)
        const GemmXSlot& S = xl[jj & 1];
        v8i a8[kGemmCB];
        int sa[kGemmCB];
#pragma unroll
        for (int c = 0; c < kGemmCB; ++c) {
          const v4i wv = wbuf[jj % kGemmWD][c];
          a8[c] = v8i{wv.x, wv.y, wv.z, wv.w, 0, 0, 0, 0};
          // weight scale byte of this step moved to byte 0 (opsel 0)
          sa[c] = (int)((uint32_t)s_cur[c][jj >> 2] >> (8 * (jj & 3)));
        }
#pragma unroll
        for (int i = 0; i < kGemmMB; ++i) {
          if (i < cur.mlive) {
            const int mb = kGemmMB * rg + i;
            const v4i lo4 = *reinterpret_cast<const v4i*>(&S.x[mb][0][lane * 16]);
            const v4i hi4 = *reinterpret_cast<const v4i*>(&S.x[mb][1][lane * 16]);
            const v8i b = v8i{lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
            const int sb = (int)(S.xs[mb * 16 + l16] >> (8 * g));
#pragma unroll
            for (int c = 0; c < kGemmCB; ++c)
              acc[c][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  a8[c], b, acc[c][i], 4, 0, 0, sa[c], 0, sb);
          }
        }
        // refill this step's weight registers with step ks + WD (of this
        // item, else of the next)
        {
          const int t = ks + kGemmWD;
          load_w(t < KS ? cur : pf, t < KS ? t : t - KS, wbuf[jj % kGemmWD]);
        }
        ring_barrier();
      }
    }
    // the next item's scale groups 0 and 1 (group 0 is already in s_nxt
    // when this item had more than one group, else in flight below)
    if (chain) {
#pragma unroll
      for (int c = 0; c < kGemmCB; ++c) s_cur[c] = s_nxt[c];
      if (KS8 == 1) load_s(nxt, 0, s_cur);
      load_s(KS8 > 1 ? nxt : none, 1, s_nxt);
    }

    // epilogue: lane holds columns 16cb + 4g .. +3 of row r0 + 16mb + l16
#pragma unroll
    for (int c = 0; c < kGemmCB; ++c) {
      const int cb = kGemmCB * cg + c;
      if (cb >= cur.ncb) continue;
      const int n = (cur.cb0 + cb) * 16 + 4 * g;
#pragma unroll
      for (int i = 0; i < kGemmMB; ++i) {
        const int mr = 16 * (kGemmMB * rg + i) + l16;
        if (i >= cur.mlive || mr >= cur.rows) continue;
        const v4f v = acc[c][i];
        const uint2 o = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
        *reinterpret_cast<uint2*>(out + (size_t)(cur.r0 + mr) * N + n) = o;
      }
    }
    item += nslot;
    cur = nxt;
    if (!chain && cur.valid) prologue(cur);
  }
}

// Load-time weight preparation (bit-exact data movement):
//   codes  w [E][N][K/2] -> wp [E][N/16][K/128][64 lanes][16 B]
//          lane l of chunk (e, cb, ks) = bytes [64ks + 16(l/16), +16) of row 16cb + l%16
//   scales s [E][N][K/32] -> sp [E][N/16][ceil(K/1024)][64 lanes][8 B]
//          byte j of lane l of (e, cb, q) = group 4(8q + j) + l/16 of row 16cb + l%16,
//          zero past the last k-step
// One wave per 1 KB chunk (codes) or 512 B unit (scales).
__global__ __launch_bounds__(256) void pack_mx_codes_kernel(const uint8_t* __restrict__ w, int N,
                                                            int K, uint8_t* __restrict__ wp) {
  const int KS = K / 128;
  const size_t per_e = (size_t)(N / 16) * KS;
  const size_t chunk = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (chunk >= per_e) return;
  const int e = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int cb = (int)(chunk / KS);
  const int ks = (int)(chunk - (size_t)cb * KS);
  const size_t row = (size_t)e * N + 16 * cb + (lane & 15);
  const uint4 v =
      *reinterpret_cast<const uint4*>(w + row * (size_t)(K / 2) + 64 * ks + 16 * (lane >> 4));
  *reinterpret_cast<uint4*>(wp + ((size_t)e * per_e + chunk) * 1024 + lane * 16) = v;
}

__global__ __launch_bounds__(256) void pack_mx_scales_kernel(const uint8_t* __restrict__ s, int N,
                                                             int K, uint8_t* __restrict__ sp) {
  const int KS = K / 128;
  const int KS8 = (KS + 7) / 8;
  const size_t per_e = (size_t)(N / 16) * KS8;
  const size_t unit = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= per_e) return;
  const int e = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int cb = (int)(unit / KS8);
  const int q = (int)(unit - (size_t)cb * KS8);
  const uint8_t* src = s + ((size_t)e * N + 16 * cb + (lane & 15)) * (size_t)(K / 32);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int ks = 8 * q + jj;
    const uint32_t b = ks < KS ? src[4 * ks + (lane >> 4)] : 0u;
    if (jj < 4) lo |= b << (8 * jj); else hi |= b << (8 * (jj - 4));
  }
  *reinterpret_cast<uint2*>(sp + ((size_t)e * per_e + unit) * 512 + lane * 8) = make_uint2(lo, hi);
}

static int launch_grouped_gemm(const uint8_t* X, const int32_t* Xs, const int32_t* ends,
                               int E_local, int A, int M_cap, int K, int N, const uint8_t* Wp,
                               const uint8_t* Sp, uint16_t* out, void* stream) {
  if (E_local < 0 || E_local > kGemmMaxE || A < 1 || M_cap < 0 || K <= 0 || N <= 0)
    return MOE_ERR_SHAPE;
  if (K % 128 != 0 || N % 128 != 0 || M_cap % 4 != 0) return MOE_ERR_ALIGN;
  // buffer ranges are 32-bit: one expert's packed weights and one 128-row
  // activation chunk must stay below 2 GiB
  if ((long long)N * K / 2 >= (1LL << 31) || (long long)kGemmBM * K >= (1LL << 31) ||
      (long long)(K / 128) * M_cap * 4 >= (1LL << 31))
    return MOE_ERR_SHAPE;
  if (E_local == 0 || M_cap == 0) return MOE_OK;
  if (!X || !Xs || !ends || !Wp || !Sp || !out) return MOE_ERR_NULL;
  // one resident block per CU; each walks its XCD's share of the item list
  const int NT = (N + kGemmBN - 1) / kGemmBN;
  const long long max_items = (long long)((M_cap + kGemmBM - 1) / kGemmBM + E_local) * NT;
  int grid = max_items < 256 ? (int)max_items : 256;
  grid = (grid + 7) & ~7;
  hipLaunchKernelGGL(grouped_mx_gemm_kernel, dim3(grid), dim3(kGemmThreads), 0,
                     (hipStream_t)stream, X, Xs, ends, E_local, A, M_cap, K, N, Wp, Sp, out);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

}  // namespace moe

extern "C" int moe_pack_mx_weights(const uint8_t* w, const uint8_t* w_scale, int E, int N, int K,
                                   uint8_t* w_packed, uint8_t* w_scale_packed, void* stream) {
  if (E < 0 || N < 0 || K <= 0 || E > 65535) return MOE_ERR_SHAPE;
  if (K % 128 != 0 || N % 16 != 0) return MOE_ERR_ALIGN;
  if (E == 0 || N == 0) return MOE_OK;
  if (!w || !w_scale || !w_packed || !w_scale_packed) return MOE_ERR_NULL;
  const size_t chunks = (size_t)(N / 16) * (K / 128);
  const size_t units = (size_t)(N / 16) * ((K / 128 + 7) / 8);
  if ((chunks + 3) / 4 > 0x7fffffffu) return MOE_ERR_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(moe::pack_mx_codes_kernel, dim3((unsigned)((chunks + 3) / 4), (unsigned)E),
                     dim3(256), 0, st, w, N, K, w_packed);
  MOE_CHECK_LAUNCH();
  hipLaunchKernelGGL(moe::pack_mx_scales_kernel, dim3((unsigned)((units + 3) / 4), (unsigned)E),
                     dim3(256), 0, st, w_scale, N, K, w_scale_packed);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_grouped_gemm1(const uint8_t* xq, const int32_t* xs, const int32_t* expert_ends,
                                 int E_local, int A, int M_cap, int H, int I,
                                 const uint8_t* w13_packed, const uint8_t* w13_scale_packed,
                                 uint16_t* gateup, void* stream) {
  if (I <= 0 || I % 64 != 0) return MOE_ERR_ALIGN;
  return moe::launch_grouped_gemm(xq, xs, expert_ends, E_local, A, M_cap, H, 2 * I, w13_packed,
                                  w13_scale_packed, gateup, stream);
}

extern "C" int moe_grouped_gemm2(const uint8_t* hq, const int32_t* hs, const int32_t* expert_ends,
                                 int E_local, int A, int M_cap, int I, int H,
                                 const uint8_t* w2_packed, const uint8_t* w2_scale_packed,
                                 uint16_t* down, void* stream) {
  return moe::launch_grouped_gemm(hq, hs, expert_ends, E_local, A, M_cap, I, H, w2_packed,
                                  w2_scale_packed, down, stream);
}
