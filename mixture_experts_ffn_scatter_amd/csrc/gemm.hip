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
// block from expert_ends (a block-wide scan of ceil(count_e/128) * N/128),
// so the grid depends only on host-known sizes and the call needs no
// device-to-host read. A persistent grid walks the list; m-tiles of one
// (expert, n-tile) are adjacent so concurrent blocks share weight tiles in
// cache. Empty experts produce no tiles and read no weights. Inside a tile,
// 16-row blocks past the expert's end issue neither loads nor MFMAs.
#include "common.h"

namespace moe {

constexpr int kGemmThreads = 256;
constexpr int kGemmBM = 128;   // rows (tokens) per tile
constexpr int kGemmBN = 128;   // output columns per tile
constexpr int kGemmMaxE = 1024;

__device__ int block_exclusive_scan_256(int v, int* tmp) {
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

__global__ __launch_bounds__(kGemmThreads) void grouped_mx_gemm_kernel(
    const uint8_t* __restrict__ X, const int32_t* __restrict__ Xs,
    const int32_t* __restrict__ expert_ends, int E_local, int A, int M_cap, int K, int N,
    const uint8_t* __restrict__ W, const uint8_t* __restrict__ Ws, uint16_t* __restrict__ out) {
  __shared__ int s_prefix[kGemmMaxE + 1];
  __shared__ int s_start[kGemmMaxE];
  __shared__ int s_end[kGemmMaxE];
  __shared__ int s_tmp[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int NT = N / kGemmBN;

  // per-expert tile counts and their exclusive scan (4 experts per thread)
  int cnt[4];
  int local_sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid * 4 + j;
    cnt[j] = 0;
    if (e < E_local) {
      int s, en;
      expert_range(expert_ends, e, A, M_cap, s, en);
      s_start[e] = s;
      s_end[e] = en;
      cnt[j] = ((en - s + kGemmBM - 1) / kGemmBM) * NT;
    }
    local_sum += cnt[j];
  }
  int run = block_exclusive_scan_256(local_sum, s_tmp);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid * 4 + j;
    if (e < E_local) s_prefix[e] = run;
    run += cnt[j];
  }
  if (tid == kGemmThreads - 1) s_prefix[E_local] = run;
  __syncthreads();
  const int total = s_prefix[E_local];

  const int wn = wid >> 1;  // wave's 64-column half of the tile
  const int wm = wid & 1;   // wave's 64-row half of the tile
  const int l16 = lane & 15;
  const int kq = lane >> 4;  // which 32-wide k slice of a 128 block this lane holds
  const size_t wrow = (size_t)K / 2;
  const size_t srow = (size_t)K / 32;

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    // expert of this tile: largest e with prefix[e] <= tile
    int lo = 0, hi = E_local - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_prefix[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int start = s_start[e], end = s_end[e];
    const int mt = (end - start + kGemmBM - 1) / kGemmBM;
    const int local = tile - s_prefix[e];
    const int n_tile = local / mt;
    const int m_tile = local - n_tile * mt;
    const int row0 = start + m_tile * kGemmBM + wm * 64;
    const int n0 = n_tile * kGemmBN + wn * 64;
    const int rows_left = end - row0;  // rows of this wave that are live (may be <= 0)

    const uint8_t* We = W + (size_t)e * N * wrow;
    const uint8_t* Wse = Ws + (size_t)e * N * srow;

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    if (rows_left > 0) {
      int nblk = (rows_left + 15) / 16;  // live 16-row blocks of this wave (1..4)
      nblk = nblk > 4 ? 4 : nblk;
      for (int k0 = 0; k0 < K; k0 += 128) {
        v4i a[4];
        int sa[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int n = n0 + nb * 16 + l16;
          a[nb] = *reinterpret_cast<const v4i*>(We + n * wrow + (k0 >> 1) + kq * 16);
          const uint32_t sw = *reinterpret_cast<const uint32_t*>(Wse + n * srow + (k0 >> 5));
          sa[nb] = (int)(sw >> (8 * kq));
        }
        v8i b[4];
        int sb[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int m = row0 + mb * 16 + l16;
          const bool ok = (mb < nblk) && (m < end);
          if (ok) {
            const uint8_t* px = X + (size_t)m * K + k0 + kq * 16;
            const v4i lo4 = *reinterpret_cast<const v4i*>(px);
            const v4i hi4 = *reinterpret_cast<const v4i*>(px + 64);
            b[mb] = v8i{lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
            const uint32_t xw = (uint32_t)Xs[(size_t)(k0 >> 7) * M_cap + m];
            sb[mb] = (int)(xw >> (8 * kq));
          } else {
            b[mb] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            sb[mb] = 127;
          }
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const v8i a8 = v8i{a[nb].x, a[nb].y, a[nb].z, a[nb].w, 0, 0, 0, 0};
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            if (mb < nblk)
              acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  a8, b[mb], acc[nb][mb], 4, 0, 0, sa[nb], 0, sb[mb]);
          }
        }
      }
      // epilogue: lane holds columns n0+16nb+4kq .. +3 of row row0+16mb+l16
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int m = row0 + mb * 16 + l16;
        if (mb >= nblk || m >= end) continue;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int n = n0 + nb * 16 + kq * 4;
          const v4f c = acc[nb][mb];
          const uint2 o = make_uint2(pack_bf16x2(c.x, c.y), pack_bf16x2(c.z, c.w));
          *reinterpret_cast<uint2*>(out + (size_t)m * N + n) = o;
        }
      }
    }
  }
}

static int launch_grouped_gemm(const uint8_t* X, const int32_t* Xs, const int32_t* ends,
                               int E_local, int A, int M_cap, int K, int N, const uint8_t* W,
                               const uint8_t* Ws, uint16_t* out, void* stream) {
  if (E_local < 0 || E_local > kGemmMaxE || A < 1 || M_cap < 0 || K <= 0 || N <= 0)
    return MOE_ERR_SHAPE;
  if (K % 128 != 0 || N % kGemmBN != 0 || M_cap % 4 != 0) return MOE_ERR_ALIGN;
  if (E_local == 0 || M_cap == 0) return MOE_OK;
  if (!X || !Xs || !ends || !W || !Ws || !out) return MOE_ERR_NULL;
  // enough blocks to fill every CU twice; each walks the device-built tile list
  const int max_tiles = ((M_cap + kGemmBM - 1) / kGemmBM + E_local) * (N / kGemmBN);
  const int grid = max_tiles < 512 ? max_tiles : 512;
  hipLaunchKernelGGL(grouped_mx_gemm_kernel, dim3(grid), dim3(kGemmThreads), 0,
                     (hipStream_t)stream, X, Xs, ends, E_local, A, M_cap, K, N, W, Ws, out);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

}  // namespace moe

extern "C" int moe_grouped_gemm1(const uint8_t* xq, const int32_t* xs, const int32_t* expert_ends,
                                 int E_local, int A, int M_cap, int H, int I, const uint8_t* w13,
                                 const uint8_t* w13_scale, uint16_t* gateup, void* stream) {
  if (I <= 0 || H <= 0) return MOE_ERR_SHAPE;
  if ((2 * I) % moe::kGemmBN != 0) return MOE_ERR_ALIGN;
  return moe::launch_grouped_gemm(xq, xs, expert_ends, E_local, A, M_cap, H, 2 * I, w13, w13_scale,
                                  gateup, stream);
}

extern "C" int moe_grouped_gemm2(const uint8_t* hq, const int32_t* hs, const int32_t* expert_ends,
                                 int E_local, int A, int M_cap, int I, int H, const uint8_t* w2,
                                 const uint8_t* w2_scale, uint16_t* down, void* stream) {
  if (I <= 0 || H <= 0) return MOE_ERR_SHAPE;
  return moe::launch_grouped_gemm(hq, hs, expert_ends, E_local, A, M_cap, I, H, w2, w2_scale, down,
                                  stream);
}
