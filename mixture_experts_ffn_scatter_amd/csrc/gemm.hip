// moe_grouped_gemm1 / moe_grouped_gemm2: grouped MX GEMMs over the live rows
// of the aligned expert layout, on gfx950 scaled MFMA.
//
//   out[m, n] = sum_k X[m, k] * W_e[n, k]      for m in [start_e, end_e)
//
// X is E4M3 with one UE8M0 byte per 32 columns (packed MN-major, four per
// int32), W_e is packed E2M1 (two per byte, low nibble = even column) with
// one E8M0 byte per 32 columns ("Blackwell DeepGEMM FusedMoE (sglang)",
// sections 2.3 / 2.5 / 3.3 and 3.8: contiguous grouped FP8 x FP4 GEMM with
// (1,32) weight scales; here the activation recipe is (1,32) as well).
// "Blackwell FP4 MoE: live-row boundary", section 2: both GEMMs take the
// int32 expert ends; rows outside [start_e, end_e) are neither read nor
// written.
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
// Scheduling: the tile list (expert, n-tile, m-tile) is rebuilt inside every
// block from expert_ends (a block-wide scan of ceil(count_e/128) * N/512),
// so the grid depends only on host-known sizes and the call needs no
// device-to-host read. A persistent grid walks the list; m-tiles of one
// (expert, n-tile) are adjacent so concurrent blocks share weight tiles in
// cache. Empty experts produce no tiles and read no weights. Inside a tile,
// 16-row blocks past the expert's end issue neither loads nor MFMAs.
#include "common.h"

namespace moe {

constexpr int kGemmThreads = 512;  // 8 waves: 2 (rows) x 4 (columns)
constexpr int kGemmBM = 128;       // rows (tokens) per tile
constexpr int kGemmBN = 512;       // output columns per tile
constexpr int kGemmBK = 128;       // k per pipeline stage (one MFMA k-step)
constexpr int kGemmStages = 3;
constexpr int kGemmMaxE = 1024;

// One pipeline stage in LDS, in MFMA fragment order so that every fragment
// read is one contiguous 1 KB ds_read_b128 per wave:
//   w[nb][lane]      16 B: weight row 16nb + lane%16, bytes [16*(lane/16), +16) of the k-step
//   x[mb][h][lane]   16 B: activation row 16mb + lane%16, k [64h + 16*(lane/16), +16)
//   ws[n], xs[m]     the packed E8M0 word (four 32-groups) of the k-step
struct __attribute__((aligned(16))) GemmStage {
  uint8_t w[kGemmBN / 16][64 * 16];
  uint8_t x[kGemmBM / 16][2][64 * 16];
  uint32_t ws[kGemmBN];
  uint32_t xs[kGemmBM];
};

// Direct global -> LDS copies (16 or 4 bytes per lane; lane i's bytes land
// at the wave-uniform LDS base in M0 plus i * size). Issued through inline
// assembly so that the compiler does not track them: its conservative
// tracking would drain the whole ring before every LDS read. Completion is
// awaited explicitly with wait_vmcnt() before the ring barrier.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}
// base: wave-uniform global address (SGPR pair); off: per-lane byte offset
__device__ __forceinline__ void lds_load16(const void* base, uint32_t off, const void* l) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(lds_addr(l)) : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(const void* base, uint32_t off, const void* l) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(off), "s"(base), "s"(lds_addr(l)) : "memory", "m0");
}

// Workgroup barrier for the LDS ring. __syncthreads() adds a release fence
// that drains every outstanding load of the wave, which would empty the
// pipeline; here each wave has already waited for its own copies of the
// stage it is about to read, so a bare s_barrier (plus completion of this
// wave's LDS reads) is enough. The memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// wait until at most N vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// the same with a wave-uniform runtime count (0..16); the immediate comes from a switch
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  switch (n) {
#define MOE_W(N) case N: wait_vmcnt<N>(); break;
    MOE_W(1) MOE_W(2) MOE_W(3) MOE_W(4) MOE_W(5) MOE_W(6) MOE_W(7) MOE_W(8)
    MOE_W(9) MOE_W(10) MOE_W(11) MOE_W(12) MOE_W(13) MOE_W(14) MOE_W(15) MOE_W(16)
#undef MOE_W
    default: wait_vmcnt<0>(); break;
  }
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

__global__ __launch_bounds__(kGemmThreads, 1) void grouped_mx_gemm_kernel(
    const uint8_t* __restrict__ X, const int32_t* __restrict__ Xs,
    const int32_t* __restrict__ expert_ends, int E_local, int A, int M_cap, int K, int N,
    const uint8_t* __restrict__ W, const int32_t* __restrict__ Wsp, uint16_t* __restrict__ out) {
  __shared__ GemmStage st[kGemmStages];
  __shared__ int s_prefix[kGemmMaxE + 1];
  __shared__ int s_tmp[kGemmThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int NT = (N + kGemmBN - 1) / kGemmBN;

  // per-expert tile counts and their exclusive scan (2 experts per thread)
  int cnt[2];
  int local_sum = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = tid * 2 + j;
    cnt[j] = 0;
    if (e < E_local) {
      int s, en;
      expert_range(expert_ends, e, A, M_cap, s, en);
      cnt[j] = ((en - s + kGemmBM - 1) / kGemmBM) * NT;
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
  const int total = s_prefix[E_local];

  const int wm = wid & 1;    // wave's 64-row half of the tile
  const int wn = wid >> 1;   // wave's 128-column quarter of the tile
  const int l16 = lane & 15;
  const int kq = lane >> 4;
  const size_t wrow = (size_t)K / 2;
  const int nk = K / kGemmBK;

  // XCD-aware order: blocks are dealt round-robin over the 8 XCDs, so
  // block b runs on XCD b % 8. Renumber so that each XCD walks a contiguous
  // run of the tile list: the n-tiles of one expert (which share its
  // activation rows) and the m-tiles of one n-tile (which share its weight
  // slice) then meet in the same L2.
  const int G = gridDim.x;
  const int vb = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
  for (int tile = vb; tile < total; tile += G) {
    int lo = 0, hi = E_local - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_prefix[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    int start, end;
    expert_range(expert_ends, e, A, M_cap, start, end);
    const int mt = (end - start + kGemmBM - 1) / kGemmBM;
    const int local = tile - s_prefix[e];
    const int n_tile = local / mt;
    const int m_tile = local - n_tile * mt;
    const int tr0 = start + m_tile * kGemmBM;   // first row of the tile
    const int tn0 = n_tile * kGemmBN;           // first column of the tile
    const uint8_t* We = W + (size_t)e * N * wrow;
    const int32_t* Wse = Wsp + (size_t)e * nk * N;   // [K/128][N] words of expert e

    // this wave's share of each stage's copies; only live data is fetched:
    //   weights: columns [tn0 + 64*wid, +64) (4 x 1 KB + 256 B of scales)
    //   activations: rows [tr0 + 16*wid, +16) (2 x 1 KB) when any is live;
    //   activation scales: waves 0,1 fetch rows [tr0 + 64*wid, +64)
    const bool w_live = tn0 + 64 * wid < N;
    const bool x_live = tr0 + 16 * wid < end;
    const bool xs_live = wid < 2 && tr0 + 64 * wid < end;
    const int loads = (w_live ? 5 : 0) + (x_live ? 2 : 0) + (xs_live ? 1 : 0);
    // per-lane byte offsets (loop-invariant); the k-step advances the
    // wave-uniform bases instead. Offsets stay below 4 GiB: a weight matrix
    // is N*K/2 bytes and an activation buffer M_cap*K bytes.
    const uint32_t ow = (uint32_t)((size_t)(tn0 + 64 * wid + l16) * wrow + kq * 16);
    const uint32_t ow_step = (uint32_t)(16 * wrow);
    const uint32_t osw = (uint32_t)(4 * (tn0 + 64 * wid + lane));
    const int mx = min(tr0 + 16 * wid + l16, end - 1);   // never a padding row
    const uint32_t ox = (uint32_t)((size_t)mx * K + kq * 16);
    const uint32_t osx = (uint32_t)(4 * min(tr0 + 64 * wid + lane, end - 1));

    auto issue = [&](int ks, GemmStage& S) {
      const int k0 = ks * kGemmBK;
      if (w_live) {
        const uint8_t* bw = We + (k0 >> 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) lds_load16(bw, ow + j * ow_step, &S.w[4 * wid + j][0]);
        lds_load4(Wse + (size_t)ks * N, osw, &S.ws[64 * wid]);
      }
      if (x_live) {
        lds_load16(X + k0, ox, &S.x[wid][0][0]);
        lds_load16(X + k0 + 64, ox, &S.x[wid][1][0]);
      }
      if (xs_live) lds_load4(Xs + (size_t)(k0 >> 7) * M_cap, osx, &S.xs[64 * wid]);
    };

    const int row0 = tr0 + wm * 64;     // this wave's first output row
    const int rows_left = end - row0;
    int nblk = rows_left <= 0 ? 0 : (rows_left + 15) / 16;
    nblk = nblk > 4 ? 4 : nblk;
    const bool c_live = tn0 + 128 * wn < N;   // N % 128 == 0: whole quarter live or dead
    if (!c_live) nblk = 0;

    v4f acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // the wave's 8 column blocks in two halves of 4, so that only 4 weight
    // fragments are live next to the 128 accumulators; activation fragments
    // are read once per half
    auto compute = [&](const GemmStage& S) {
      if (nblk == 0) return;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        v4i a[4];
        int sa[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int nb = 8 * wn + 4 * hb + j;
          a[j] = *reinterpret_cast<const v4i*>(&S.w[nb][lane * 16]);
          sa[j] = (int)(S.ws[nb * 16 + l16] >> (8 * kq));
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          if (mb < nblk) {
            const v4i lo4 = *reinterpret_cast<const v4i*>(&S.x[4 * wm + mb][0][lane * 16]);
            const v4i hi4 = *reinterpret_cast<const v4i*>(&S.x[4 * wm + mb][1][lane * 16]);
            const v8i b = v8i{lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
            const int sb = (int)(S.xs[(4 * wm + mb) * 16 + l16] >> (8 * kq));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const v8i a8 = v8i{a[j].x, a[j].y, a[j].z, a[j].w, 0, 0, 0, 0};
              acc[4 * hb + j][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  a8, b, acc[4 * hb + j][mb], 4, 0, 0, sa[j], 0, sb);
            }
          }
        }
      }
    };

    // the ring: keep kGemmStages-1 stages in flight; at step ks refill the
    // slot consumed at step ks-1, wait for stage ks, compute, and fence
    // before that slot is refilled again
#pragma unroll
    for (int s = 0; s < kGemmStages - 1; ++s)
      if (s < nk) issue(s, st[s]);
    for (int ks = 0; ks < nk; ++ks) {
      const int nxt = ks + kGemmStages - 1;
      if (nxt < nk) {
        issue(nxt, st[nxt % kGemmStages]);
        wait_vmcnt_dyn((kGemmStages - 1) * loads);
      } else {
        wait_vmcnt_dyn((nk - 1 - ks) * loads);
      }
      ring_barrier();
      compute(st[ks % kGemmStages]);
      ring_barrier();
    }

    // epilogue: lane holds columns n0+16nb+4kq .. +3 of row row0+16mb+l16
    const int n0 = tn0 + wn * 128;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = row0 + mb * 16 + l16;
      if (mb >= nblk || m >= end) continue;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int n = n0 + nb * 16 + kq * 4;
        const v4f c = acc[nb][mb];
        const uint2 o = make_uint2(pack_bf16x2(c.x, c.y), pack_bf16x2(c.z, c.w));
        *reinterpret_cast<uint2*>(out + (size_t)m * N + n) = o;
      }
    }
  }
}

static int launch_grouped_gemm(const uint8_t* X, const int32_t* Xs, const int32_t* ends,
                               int E_local, int A, int M_cap, int K, int N, const uint8_t* W,
                               const int32_t* Ws, uint16_t* out, void* stream) {
  if (E_local < 0 || E_local > kGemmMaxE || A < 1 || M_cap < 0 || K <= 0 || N <= 0)
    return MOE_ERR_SHAPE;
  if (K % 128 != 0 || N % 128 != 0 || M_cap % 4 != 0) return MOE_ERR_ALIGN;
  // per-lane copy offsets are 32-bit: one expert's weights and the whole
  // activation buffer must each stay below 4 GiB
  if ((long long)N * K / 2 >= (1LL << 32) || (long long)M_cap * K >= (1LL << 32))
    return MOE_ERR_SHAPE;
  if (E_local == 0 || M_cap == 0) return MOE_OK;
  if (!X || !Xs || !ends || !W || !Ws || !out) return MOE_ERR_NULL;
  // one resident block per CU (LDS-limited); each walks the device-built tile list
  const int max_tiles = ((M_cap + kGemmBM - 1) / kGemmBM + E_local) * ((N + kGemmBN - 1) / kGemmBN);
  const int grid = max_tiles < 256 ? max_tiles : 256;
  hipLaunchKernelGGL(grouped_mx_gemm_kernel, dim3(grid), dim3(kGemmThreads), 0,
                     (hipStream_t)stream, X, Xs, ends, E_local, A, M_cap, K, N, W, Ws, out);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

// E8M0 weight scales, row-major bytes [E][N][K/32] -> packed words laid out
// MN-major [E][K/128][N] (word c of row n holds groups 4c..4c+3, byte j =
// group 4c+j). One word per thread; consecutive threads write consecutive n.
__global__ __launch_bounds__(256) void pack_weight_scales_kernel(const uint8_t* __restrict__ s,
                                                                 int N, int K,
                                                                 int32_t* __restrict__ out) {
  const int e = blockIdx.z;
  const int c = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(s + ((size_t)e * N + n) * (K / 32) + 4 * c);
  out[((size_t)e * (K / 128) + c) * N + n] = (int32_t)w;
}

}  // namespace moe

extern "C" int moe_pack_weight_scales(const uint8_t* w_scale, int E, int N, int K,
                                      int32_t* w_scale_packed, void* stream) {
  if (E < 0 || N < 0 || K <= 0) return MOE_ERR_SHAPE;
  if (K % 128 != 0) return MOE_ERR_ALIGN;
  if (E == 0 || N == 0) return MOE_OK;
  if (!w_scale || !w_scale_packed) return MOE_ERR_NULL;
  if (K / 128 > 65535 || E > 65535) return MOE_ERR_SHAPE;
  dim3 grid((N + 255) / 256, K / 128, E);
  hipLaunchKernelGGL(moe::pack_weight_scales_kernel, grid, dim3(256), 0, (hipStream_t)stream,
                     w_scale, N, K, w_scale_packed);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_grouped_gemm1(const uint8_t* xq, const int32_t* xs, const int32_t* expert_ends,
                                 int E_local, int A, int M_cap, int H, int I, const uint8_t* w13,
                                 const int32_t* w13_scale_packed, uint16_t* gateup, void* stream) {
  if (I <= 0 || H <= 0) return MOE_ERR_SHAPE;
  return moe::launch_grouped_gemm(xq, xs, expert_ends, E_local, A, M_cap, H, 2 * I, w13,
                                  w13_scale_packed, gateup, stream);
}

extern "C" int moe_grouped_gemm2(const uint8_t* hq, const int32_t* hs, const int32_t* expert_ends,
                                 int E_local, int A, int M_cap, int I, int H, const uint8_t* w2,
                                 const int32_t* w2_scale_packed, uint16_t* down, void* stream) {
  if (I <= 0 || H <= 0) return MOE_ERR_SHAPE;
  return moe::launch_grouped_gemm(hq, hs, expert_ends, E_local, A, M_cap, I, H, w2,
                                  w2_scale_packed, down, stream);
}
