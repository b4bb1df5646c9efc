// History coordinate rewrite: C[0:n, 0:k+] <- C[0:n, 0:k] H_top, in place.
//
// Page "iS-KV: Online Low-Rank KV Cache Compression via Block-Incremental
// SVD", section "Block-Incremental Decoding Updates", equation for U+: every
// stored row is re-expressed in the new basis ([U 0; 0 I] G, here applied to
// C = U Sigma as C H_top, see k_core.hip). Columns k+ .. r-1 are written as
// zero, so every stored row is always r wide and clean.
//
// This is the HBM stream of a fold: each row is read once and written once.
// A workgroup owns a tile of rows, so the in-place update is race free (the
// tile is staged in LDS before any row of it is written).
#include "iskv_internal.hpp"

namespace iskv {

namespace {

constexpr int TILE = 64;  // rows per workgroup iteration

// XK (0 keys, 1 values) is a template constant so that every access to the
// kernel arguments has a constant offset.
template <typename TC, int XK>
__device__ __forceinline__ void rewrite_body(const RewriteArgs &a, float *sm) {
  const Stream &X = a.X[XK];
  const int k = a.k[XK], kp = a.kp[XK], r = a.r[XK];
  if (a.n <= 0 || k <= 0) return;
  const int ldx = k + 1;  // padded row stride of the staged tile
  float *Hs = sm;                    // k x kp
  float *Xs = sm + (size_t)k * kp;   // TILE x ldx
  const int u = a.u0 + blockIdx.y;
  const float *Ht = X.Htop + (size_t)u * r * r;
  for (int idx = threadIdx.x; idx < k * kp; idx += NT) {
    const int i = idx / kp, j = idx - i * kp;
    Hs[idx] = Ht[(size_t)i * r + j];
  }
  TC *C = (TC *)X.C + (size_t)u * a.ncap * r;
  const int row_l = threadIdx.x & (TILE - 1);
  const int cg = threadIdx.x / TILE;  // 4 column groups
  for (int t0 = blockIdx.x * TILE; t0 < a.n; t0 += gridDim.x * TILE) {
    const int nrow = min(TILE, a.n - t0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < nrow * k; idx += NT) {
      const int i = idx / k, j = idx - i * k;
      Xs[i * ldx + j] = ldf<TC>(C, (size_t)(t0 + i) * r + j);
    }
    __syncthreads();
    if (row_l < nrow) {
      const float *x = Xs + row_l * ldx;
      TC *crow = C + (size_t)(t0 + row_l) * r;
      for (int j0 = cg; j0 < r; j0 += 4 * 8) {
        float acc[8];
#pragma unroll
        for (int z = 0; z < 8; z++) acc[z] = 0.f;
        for (int i = 0; i < k; i++) {
          const float xv = x[i];
#pragma unroll
          for (int z = 0; z < 8; z++) {
            const int j = j0 + 4 * z;
            if (j < kp) acc[z] += xv * Hs[i * kp + j];
          }
        }
#pragma unroll
        for (int z = 0; z < 8; z++) {
          const int j = j0 + 4 * z;
          if (j < r) stf<TC>(crow, j, (j < kp) ? acc[z] : 0.f);
        }
      }
    }
  }
}

template <typename TC>
__global__ void __launch_bounds__(NT) k_rewrite_vec(const RewriteArgs a) {
  extern __shared__ float sm[];
  if (blockIdx.z == 0)
    rewrite_body<TC, 0>(a, sm);
  else
    rewrite_body<TC, 1>(a, sm);
}

}  // namespace

hipError_t launch_rewrite(const RewriteArgs &a, int nunits, int coord_bf16, hipStream_t s) {
  if (a.n <= 0 || nunits <= 0) return hipSuccess;
  size_t lds = 0;
  for (int x = 0; x < 2; x++) {
    const size_t l = sizeof(float) * ((size_t)a.k[x] * a.kp[x] + (size_t)TILE * (a.k[x] + 1));
    if (l > lds) lds = l;
  }
  int tiles = (a.n + TILE - 1) / TILE;
  if (tiles > 64) tiles = 64;
  dim3 grid(tiles, nunits, 2);
  if (coord_bf16) {
    hipError_t e = hipFuncSetAttribute((const void *)k_rewrite_vec<uint16_t>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_rewrite_vec<uint16_t>, grid, dim3(NT), lds, s, a);
  } else {
    hipError_t e = hipFuncSetAttribute((const void *)k_rewrite_vec<float>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_rewrite_vec<float>, grid, dim3(NT), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace iskv
