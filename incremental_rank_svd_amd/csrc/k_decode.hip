// Single-token decode attention over the compressed cache.
//
// For a history row i, K~_i = C_K[i] B_K^T (section "Reconstruction and
// Storage" of the iS-KV page), so its score is
//     s_i = scale * K~_i . q = C_K[i] . q'   with   q' = scale * B_K^T q,
// and the weighted history values are (sum_i p_i C_V[i]) B_V^T. The window
// rows are used as stored. Softmax runs over history and window together,
// split over chunks of history rows and merged by log-sum-exp.
//
// One launch, grid (history chunks + 1, units):
//   - a history block computes q' for its unit, then (max, sum, o' = sum p C_V)
//     over its chunk of rows; the extra block does the same over the window
//     rows with the raw query;
//   - the last block of a unit to finish (atomic ticket, reset by that block)
//     merges the partials by log-sum-exp, applies B_V^T, adds the window part
//     and normalises. The output stays fp32 (the compute type).
#include "iskv_internal.hpp"

namespace iskv {

namespace {

constexpr int MAXG = 8;  // query heads per kv head handled by one workgroup
constexpr int QS_FLOATS = (NT * MAXG > MAXG * D) ? NT * MAXG : MAXG * D;

__device__ __forceinline__ void unit_coords(const DecodeArgs &a, int ul, int &li, int &bi, int &h) {
  h = ul % a.L.kvh;
  const int t = ul / a.L.kvh;
  bi = t % a.L.batch;
  li = t / a.L.batch;
}

// block-wide max/sum of one value per head; red must hold 4 * MAXG floats
__device__ __forceinline__ void block_reduce_heads(float *vals, int g, float *red, bool is_max) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  for (int hh = 0; hh < g; hh++) {
    float v = is_max ? max64(vals[hh]) : sum64(vals[hh]);
    if (l == 0) red[w * MAXG + hh] = v;
  }
  __syncthreads();
  for (int hh = 0; hh < g; hh++) {
    const float a0 = red[hh], a1 = red[MAXG + hh], a2 = red[2 * MAXG + hh], a3 = red[3 * MAXG + hh];
    vals[hh] = is_max ? fmaxf(fmaxf(a0, a1), fmaxf(a2, a3)) : (a0 + a1) + (a2 + a3);
  }
  __syncthreads();
}

// log-sum-exp merge of a unit's chunk partials and window part; osm must
// hold MAXG * D floats of LDS
__device__ void merge_unit(const DecodeArgs &a, int ul, int u, float *osm) {
  __shared__ float wsc[MAXG][4];  // M, L, window factor
  int li, bi, h;
  unit_coords(a, ul, li, bi, h);
  const int g = a.L.g, rV = a.L.X[1].r, kV = a.kV;
  const int stride = 2 + rV;
  const float *part = a.L.part + (size_t)u * a.L.nchunk_max * g * stride;
  const float *wp = a.L.wpart + (size_t)u * g * (2 + D);
  const int tid = threadIdx.x;
  if (tid < g) {
    float M = wp[tid * (2 + D)];
    for (int c = 0; c < a.nchunk; c++) M = fmaxf(M, part[((size_t)c * g + tid) * stride]);
    float L = (wp[tid * (2 + D) + 1] > 0.f) ? wp[tid * (2 + D) + 1] * __expf(wp[tid * (2 + D)] - M) : 0.f;
    for (int c = 0; c < a.nchunk; c++) {
      const float lc = part[((size_t)c * g + tid) * stride + 1];
      if (lc > 0.f) L += lc * __expf(part[((size_t)c * g + tid) * stride] - M);
    }
    wsc[tid][0] = M;
    wsc[tid][1] = L;
    wsc[tid][2] = (wp[tid * (2 + D) + 1] > 0.f) ? __expf(wp[tid * (2 + D)] - M) : 0.f;
  }
  __syncthreads();
  for (int idx = tid; idx < g * kV; idx += NT) {
    const int hh = idx / kV, j = idx - hh * kV;
    const float M = wsc[hh][0];
    float s = 0.f;
    for (int c = 0; c < a.nchunk; c++) {
      const float *pc = part + ((size_t)c * g + hh) * stride;
      if (pc[1] > 0.f) s += __expf(pc[0] - M) * pc[2 + j];
    }
    osm[hh * D + j] = s;
  }
  __syncthreads();
  const float *Bt = a.L.X[1].Bt + (size_t)u * rV * D;
  float *out = (float *)a.out + (((size_t)bi * a.nl_in + a.lrel0 + li) * a.L.qh + (size_t)h * g) * D;
  for (int idx = tid; idx < g * D; idx += NT) {
    const int hh = idx / D, t = idx - hh * D;
    float s = 0.f;
    for (int j = 0; j < kV; j++) s += osm[hh * D + j] * Bt[(size_t)j * D + t];
    s += wsc[hh][2] * wp[hh * (2 + D) + 2 + t];
    out[idx] = s / wsc[hh][1];
  }
}

template <typename TC, typename TK>
__global__ void __launch_bounds__(NT) k_decode(const DecodeArgs a) {
  extern __shared__ float sm[];
  const int ul = blockIdx.y;
  const int u = a.u0 + ul;
  const int g = a.L.g;
  const int tid = threadIdx.x;
  float *red = sm;                 // 4 * MAXG
  float *qs = sm + 4 * MAXG;       // g x D (window) or g x kK (history); later nz x g x width
  float *ss = qs + QS_FLOATS;      // g x rows (rows <= chunk)
  const int ch = blockIdx.x;
  const bool window = (ch == a.nchunk);
  int rows, row0 = 0;
  if (window) {
    rows = a.e;
  } else {
    row0 = ch * a.L.chunk;
    rows = min(a.L.chunk, a.n - row0);
  }
  const int ldq = window ? D : a.kK;
  // query vectors
  if (window) {
    int li, bi, h;
    unit_coords(a, ul, li, bi, h);
    const TK *q = (const TK *)a.q + (((size_t)bi * a.nl_in + a.lrel0 + li) * a.L.qh + (size_t)h * g) * D;
    for (int idx = tid; idx < g * D; idx += NT) qs[idx] = a.scale * ldf<TK>(q, idx);
  } else {
    // q' = scale * B_K^T q for the g heads of this kv head (16 lanes per dot)
    int li, bi, h;
    unit_coords(a, ul, li, bi, h);
    const TK *q = (const TK *)a.q + (((size_t)bi * a.nl_in + a.lrel0 + li) * a.L.qh + (size_t)h * g) * D;
    const float *Bt = a.L.X[0].Bt + (size_t)u * a.L.X[0].r * D;
    const int lane = tid & 15, grp = tid >> 4;
    for (int pj = grp; pj < g * a.kK; pj += 16) {
      const int hh = pj / a.kK, jj = pj - hh * a.kK;
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < 8; t++)
        s += Bt[(size_t)jj * D + lane * 8 + t] * ldf<TK>(q, (size_t)hh * D + lane * 8 + t);
      s = sum16(s);
      if (lane == 0) qs[hh * a.kK + jj] = a.scale * s;
    }
  }
  __syncthreads();
  // scores: one thread per row
  float mx[MAXG];
#pragma unroll
  for (int hh = 0; hh < MAXG; hh++) mx[hh] = -INFINITY;
  if (window) {
    const TK *kr = (const TK *)a.L.X[0].ring + (size_t)u * a.L.rcap * D;
    for (int i = tid; i < rows; i += NT) {
      int pos = a.head + i;
      if (pos >= a.L.rcap) pos -= a.L.rcap;
      float s[MAXG];
#pragma unroll
      for (int hh = 0; hh < MAXG; hh++) s[hh] = 0.f;
      for (int t = 0; t < D; t++) {
        const float x = ldf<TK>(kr, (size_t)pos * D + t);
#pragma unroll
        for (int hh = 0; hh < MAXG; hh++)
          if (hh < g) s[hh] += x * qs[hh * D + t];
      }
#pragma unroll
      for (int hh = 0; hh < MAXG; hh++)
        if (hh < g) {
          ss[hh * a.L.chunk + i] = s[hh];
          mx[hh] = fmaxf(mx[hh], s[hh]);
        }
    }
  } else {
    const int rK = a.L.X[0].r;
    const TC *ck = (const TC *)a.L.X[0].C + ((size_t)u * a.L.ncap + row0) * rK;
    for (int i = tid; i < rows; i += NT) {
      float s[MAXG];
#pragma unroll
      for (int hh = 0; hh < MAXG; hh++) s[hh] = 0.f;
      for (int j = 0; j < a.kK; j++) {
        const float x = ldf<TC>(ck, (size_t)i * rK + j);
#pragma unroll
        for (int hh = 0; hh < MAXG; hh++)
          if (hh < g) s[hh] += x * qs[hh * ldq + j];
      }
#pragma unroll
      for (int hh = 0; hh < MAXG; hh++)
        if (hh < g) {
          ss[hh * a.L.chunk + i] = s[hh];
          mx[hh] = fmaxf(mx[hh], s[hh]);
        }
    }
  }
  block_reduce_heads(mx, g, red, true);
  float sum[MAXG];
#pragma unroll
  for (int hh = 0; hh < MAXG; hh++) sum[hh] = 0.f;
  for (int i = tid; i < rows; i += NT) {
#pragma unroll
    for (int hh = 0; hh < MAXG; hh++)
      if (hh < g) {
        const float pv = __expf(ss[hh * a.L.chunk + i] - mx[hh]);
        ss[hh * a.L.chunk + i] = pv;
        sum[hh] += pv;
      }
  }
  block_reduce_heads(sum, g, red, false);  // includes a barrier: ss is complete
  // weighted values: thread -> (column j, row slice z)
  const int width = window ? D : a.kV;
  const int nz = width > 0 ? NT / width : 0;
  float *acc_sm = qs;  // reuse: nz x g x width (<= NT * MAXG floats)
  float acc[MAXG];
#pragma unroll
  for (int hh = 0; hh < MAXG; hh++) acc[hh] = 0.f;
  const int j = width > 0 ? tid % width : 0;
  const int z = width > 0 ? tid / width : 0;
  if (width > 0 && z < nz) {
    if (window) {
      const TK *vr = (const TK *)a.L.X[1].ring + (size_t)u * a.L.rcap * D;
      for (int i = z; i < rows; i += nz) {
        int pos = a.head + i;
        if (pos >= a.L.rcap) pos -= a.L.rcap;
        const float x = ldf<TK>(vr, (size_t)pos * D + j);
#pragma unroll
        for (int hh = 0; hh < MAXG; hh++)
          if (hh < g) acc[hh] += ss[hh * a.L.chunk + i] * x;
      }
    } else {
      const int rV = a.L.X[1].r;
      const TC *cv = (const TC *)a.L.X[1].C + ((size_t)u * a.L.ncap + row0) * rV;
      for (int i = z; i < rows; i += nz) {
        const float x = ldf<TC>(cv, (size_t)i * rV + j);
#pragma unroll
        for (int hh = 0; hh < MAXG; hh++)
          if (hh < g) acc[hh] += ss[hh * a.L.chunk + i] * x;
      }
    }
  }
  __syncthreads();
  if (width > 0 && z < nz) {
#pragma unroll
    for (int hh = 0; hh < MAXG; hh++)
      if (hh < g) acc_sm[((size_t)z * g + hh) * width + j] = acc[hh];
  }
  __syncthreads();
  float *dst;
  int stride;
  if (window) {
    dst = a.L.wpart + (size_t)u * g * (2 + D);
    stride = 2 + D;
  } else {
    stride = 2 + a.L.X[1].r;
    dst = a.L.part + ((size_t)u * a.L.nchunk_max + ch) * g * stride;
  }
  for (int idx = tid; idx < g * width; idx += NT) {
    const int hh = idx / width, jj = idx - hh * width;
    float s = 0.f;
    for (int zz = 0; zz < nz; zz++) s += acc_sm[((size_t)zz * g + hh) * width + jj];
    dst[hh * stride + 2 + jj] = s;
  }
  if (tid < g) {
    dst[tid * stride + 0] = rows > 0 ? mx[tid] : -INFINITY;
    dst[tid * stride + 1] = rows > 0 ? sum[tid] : 0.f;
  }
  // ---- last block of the unit merges ------------------------------------
  __threadfence();  // this block's partial is visible device-wide before its ticket
  __syncthreads();
  int *flag = (int *)red;
  if (tid == 0) {
    const unsigned t = atomicAdd(a.L.ticket + u, 1u);
    flag[0] = (t == (unsigned)a.nchunk) ? 1 : 0;
  }
  __syncthreads();
  if (!flag[0]) return;
  __threadfence();
  merge_unit(a, ul, u, qs);
  if (tid == 0) a.L.ticket[u] = 0u;
}

template <typename TC, typename TK>
hipError_t launch_decode_t(const DecodeArgs &a, int nunits, hipStream_t s) {
  const size_t lds = sizeof(float) * (4 * MAXG + QS_FLOATS + (size_t)MAXG * a.L.chunk);
  hipError_t e = hipFuncSetAttribute((const void *)k_decode<TC, TK>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_decode<TC, TK>), dim3(a.nchunk + 1, nunits), dim3(NT), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  const int nunits = a.L.batch * a.nl * a.L.kvh;
  if (a.L.coord_bf16 && a.L.kv_bf16) return launch_decode_t<uint16_t, uint16_t>(a, nunits, s);
  if (a.L.coord_bf16) return launch_decode_t<uint16_t, float>(a, nunits, s);
  if (a.L.kv_bf16) return launch_decode_t<float, uint16_t>(a, nunits, s);
  return launch_decode_t<float, float>(a, nunits, s);
}

}  // namespace iskv
