// Small kernels: window ingest, reconstruction, zero fill, ring copies.
#include "iskv_internal.hpp"

namespace iskv {

namespace {

// Copy nrows new rows per unit into the window ring (section "Architecture
// Overview": the most recent rows are kept exactly). blockIdx.y selects K/V.
// A row is moved by words_per_row consecutive threads (16-byte words when
// the source is 16-byte aligned), so the index arithmetic is per row.
template <typename W>
__global__ void __launch_bounds__(NT) k_ingest(const IngestArgs a, int words_per_row) {
  const W *src = (const W *)a.src[blockIdx.y];
  W *ring = (W *)a.ring[blockIdx.y];
  const int rows = a.batch * a.nl * a.kvh * a.nrows;
  const int rows_per_blk = NT / words_per_row;  // words_per_row divides NT
  const int wd = threadIdx.x % words_per_row, rl = threadIdx.x / words_per_row;
  for (int t = blockIdx.x * rows_per_blk + rl; t < rows; t += gridDim.x * rows_per_blk) {
    int x = t;
    const int i = x % a.nrows;
    x /= a.nrows;
    const int h = x % a.kvh;
    x /= a.kvh;
    const int li = x % a.nl;
    const int bi = x / a.nl;
    const size_t s_row = (((size_t)bi * a.nl_in + a.lrel0 + li) * a.kvh + h) * a.nrows + i;
    const size_t u = (size_t)a.u0 + ((size_t)li * a.batch + bi) * a.kvh + h;
    int pos = a.pos + i;
    if (pos >= a.rcap) pos -= a.rcap;
    ring[(u * a.rcap + pos) * words_per_row + wd] = src[s_row * words_per_row + wd];
  }
}

// Fixed-basis fold ([iS-KV] Ablation Study, "keeping bases fixed"): the b
// oldest window rows F are stored as their coordinates F B in the kept basis
// (zero beyond the rank); rank, basis and sigma stay; the discarded energy is
// ||F||^2 - ||F B||^2, the part of F outside the basis. F and B go through LDS.
template <typename TK, typename TC, int XK>
__device__ __forceinline__ void project_body(const FoldArgs &a, float *sm) {
  const Stream &X = a.X[XK];
  const int k = a.k[XK], r = a.r[XK], b = a.b;
  const int u = a.u0 + blockIdx.x;
  float *Bs = sm;                  // k x D
  float *Fs = sm + (size_t)k * D;  // b x D
  float *red = Fs + (size_t)b * D; // NT / 64 partial sums
  const float *Bt = X.Bt + (size_t)u * r * D;
  const TK *ring = (const TK *)X.ring + (size_t)u * a.rcap * D;
  for (int idx = threadIdx.x; idx < k * D; idx += NT) Bs[idx] = Bt[idx];
  for (int idx = threadIdx.x; idx < b * D; idx += NT) {
    const int i = idx / D, t = idx - i * D;
    int pos = a.head + i;
    if (pos >= a.rcap) pos -= a.rcap;
    Fs[idx] = ldf<TK>(ring, (size_t)pos * D + t);
  }
  __syncthreads();
  TC *C = (TC *)X.C + (size_t)u * X.cstride + (size_t)a.n * r;
  float lost = 0.f;
  for (int idx = threadIdx.x; idx < b * r; idx += NT) {
    const int i = idx / r, j = idx - i * r;
    float y = 0.f;
    if (j < k) {
      const float *f = Fs + (size_t)i * D, *bj = Bs + (size_t)j * D;
      for (int t = 0; t < D; t++) y += f[t] * bj[t];
    }
    stf<TC>(C, (size_t)i * r + j, y);
    lost -= y * y;
  }
  for (int idx = threadIdx.x; idx < b * D; idx += NT) lost += Fs[idx] * Fs[idx];
  lost = sum64(lost);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = lost;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < NT / 64; w++) t += red[w];
    X.disc[u] = t;
    X.sweeps[u] = 0;
  }
}

template <typename TK, typename TC>
__global__ void __launch_bounds__(NT) k_project(const FoldArgs a) {
  extern __shared__ float sm[];
  if (blockIdx.y == 0)
    project_body<TK, TC, 0>(a, sm);
  else
    project_body<TK, TC, 1>(a, sm);
}

// X~ = [C B^T ; window] for one unit (section "Reconstruction and Storage").
template <typename TC, typename TK>
__global__ void __launch_bounds__(NT) k_reconstruct(const float *Bt, const TC *C, const TK *ring,
                                                    int r, int n, int k, int e, int head, int rcap,
                                                    float *out) {
  const int row = blockIdx.x;
  if (row < n) {
    for (int t = threadIdx.x; t < D; t += NT) {
      float s = 0.f;
      for (int j = 0; j < k; j++) s += ldf<TC>(C, (size_t)row * r + j) * Bt[(size_t)j * D + t];
      out[(size_t)row * D + t] = s;
    }
  } else {
    int pos = head + (row - n);
    if (pos >= rcap) pos -= rcap;
    for (int t = threadIdx.x; t < D; t += NT) out[(size_t)row * D + t] = ldf<TK>(ring, (size_t)pos * D + t);
  }
}

// int8 storage: history row = (codes * scale) Sigma B^T
__global__ void __launch_bounds__(NT) k_reconstruct_i8(const float *Bt, const int8_t *C, const float *cs,
                                                       const float *sig, const uint16_t *ring, int r, int n,
                                                       int k, int e, int head, int rcap, float *out) {
  const int row = blockIdx.x;
  if (row < n) {
    const float sc = cs[row];
    for (int t = threadIdx.x; t < D; t += NT) {
      float s = 0.f;
      for (int j = 0; j < k; j++) s += ((float)C[(size_t)row * r + j] * sc) * sig[j] * Bt[(size_t)j * D + t];
      out[(size_t)row * D + t] = s;
    }
  } else {
    int pos = head + (row - n);
    if (pos >= rcap) pos -= rcap;
    for (int t = threadIdx.x; t < D; t += NT) out[(size_t)row * D + t] = bf2f(ring[(size_t)pos * D + t]);
  }
}

__global__ void k_zero(uint32_t *p, size_t nwords) {
  for (size_t i = (size_t)blockIdx.x * NT + threadIdx.x; i < nwords; i += (size_t)gridDim.x * NT) p[i] = 0u;
}

// Window rows between the ring (starting at head, wrapping) and a dense buffer.
__global__ void k_ring_copy(uint8_t *ring, uint8_t *dense, int e, int head, int rcap, int row_bytes,
                            int to_ring) {
  const int i = blockIdx.x;
  int pos = head + i;
  if (pos >= rcap) pos -= rcap;
  for (int t = threadIdx.x; t < row_bytes; t += NT) {
    if (to_ring)
      ring[(size_t)pos * row_bytes + t] = dense[(size_t)i * row_bytes + t];
    else
      dense[(size_t)i * row_bytes + t] = ring[(size_t)pos * row_bytes + t];
  }
}

}  // namespace

template <typename TK, typename TC>
hipError_t launch_project_t(const FoldArgs &a, int nunits, hipStream_t s) {
  const int kmax = a.k[0] > a.k[1] ? a.k[0] : a.k[1];
  const size_t lds = sizeof(float) * ((size_t)(kmax + a.b) * D + NT / 64);
  hipError_t e = hipFuncSetAttribute((const void *)k_project<TK, TC>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_project<TK, TC>), dim3(nunits, 2), dim3(NT), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_project(const FoldArgs &a, int nunits, int kv_bf16, int coord_bf16, hipStream_t s) {
  if (kv_bf16 && coord_bf16) return launch_project_t<uint16_t, uint16_t>(a, nunits, s);
  if (kv_bf16) return launch_project_t<uint16_t, float>(a, nunits, s);
  if (coord_bf16) return launch_project_t<float, uint16_t>(a, nunits, s);
  return launch_project_t<float, float>(a, nunits, s);
}

hipError_t launch_ingest(const IngestArgs &a, int kv_bf16, hipStream_t s) {
  const int row_bytes = D * (kv_bf16 ? 2 : 4);
  const int rows = a.batch * a.nl * a.kvh * a.nrows;
  if (rows <= 0) return hipSuccess;
  const bool wide = (((uintptr_t)a.src[0] | (uintptr_t)a.src[1]) & 15) == 0;
  const int wpr = row_bytes / (wide ? 16 : 4);
  size_t blocks = ((size_t)rows * wpr + NT - 1) / NT;
  if (blocks > 4096) blocks = 4096;
  if (wide)
    hipLaunchKernelGGL(k_ingest<uint4>, dim3((unsigned)blocks, 2), dim3(NT), 0, s, a, wpr);
  else
    hipLaunchKernelGGL(k_ingest<uint32_t>, dim3((unsigned)blocks, 2), dim3(NT), 0, s, a, wpr);
  return hipGetLastError();
}

hipError_t launch_reconstruct(const Layout &L, int which, int u, int n, int k, int e, int head,
                              float *out, hipStream_t s) {
  const Stream &X = L.X[which];
  const int rows = n + e;
  if (rows == 0) return hipSuccess;
  const float *Bt = X.Bt + (size_t)u * X.r * D;
  const size_t coff = (size_t)u * X.cstride;
  const size_t roff = (size_t)u * L.rcap * D;
  if (L.coord_i8) {
    hipLaunchKernelGGL(k_reconstruct_i8, dim3(rows), dim3(NT), 0, s, Bt, (const int8_t *)X.C + coff,
                       X.cs + (size_t)u * cs_stride(L.ncap), X.sig + (size_t)u * X.r, (const uint16_t *)X.ring + roff, X.r,
                       n, k, e, head, L.rcap, out);
    return hipGetLastError();
  }
  if (L.coord_bf16 && L.kv_bf16)
    hipLaunchKernelGGL((k_reconstruct<uint16_t, uint16_t>), dim3(rows), dim3(NT), 0, s, Bt,
                       (const uint16_t *)X.C + coff, (const uint16_t *)X.ring + roff, X.r, n, k, e, head,
                       L.rcap, out);
  else if (L.coord_bf16)
    hipLaunchKernelGGL((k_reconstruct<uint16_t, float>), dim3(rows), dim3(NT), 0, s, Bt,
                       (const uint16_t *)X.C + coff, (const float *)X.ring + roff, X.r, n, k, e, head,
                       L.rcap, out);
  else if (L.kv_bf16)
    hipLaunchKernelGGL((k_reconstruct<float, uint16_t>), dim3(rows), dim3(NT), 0, s, Bt,
                       (const float *)X.C + coff, (const uint16_t *)X.ring + roff, X.r, n, k, e, head,
                       L.rcap, out);
  else
    hipLaunchKernelGGL((k_reconstruct<float, float>), dim3(rows), dim3(NT), 0, s, Bt,
                       (const float *)X.C + coff, (const float *)X.ring + roff, X.r, n, k, e, head,
                       L.rcap, out);
  return hipGetLastError();
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  size_t blocks = (words + NT - 1) / NT;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(NT), 0, s, (uint32_t *)p, words);
  return hipGetLastError();
}

hipError_t launch_ring_copy(const Layout &L, int which, int u, int e, int head, void *dst,
                            const void *src, int to_ring, hipStream_t s) {
  if (e <= 0) return hipSuccess;
  const int row_bytes = D * (L.kv_bf16 ? 2 : 4);
  uint8_t *ring = (uint8_t *)L.X[which].ring + (size_t)u * L.rcap * row_bytes;
  uint8_t *dense = (uint8_t *)(to_ring ? src : dst);
  hipLaunchKernelGGL(k_ring_copy, dim3(e), dim3(NT), 0, s, ring, dense, e, head, L.rcap, row_bytes,
                     to_ring);
  return hipGetLastError();
}

}  // namespace iskv
