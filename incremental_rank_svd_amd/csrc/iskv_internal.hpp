// Internal declarations of the gfx950 iS-KV library: state layout in HBM,
// kernel argument blocks, small device helpers and the kernel launchers.
// Every kernel is hand-written HIP for gfx950 (64-wide wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace iskv {

constexpr int D = 128;         // head dimension
constexpr int NT = 256;        // threads per workgroup (4 wavefronts)
// update modes, same values as ISKV_MODE_* in iskv.h
constexpr int MODE_JOINT = 0, MODE_FIXED_COORDS = 1, MODE_FIXED_BASIS = 2;
constexpr int SWEEP_CAP = 40;  // core SVD sweep cap (flagged when reached)

constexpr uint32_t FLAG_SWEEP_CAP = 0x1u;
constexpr uint32_t FLAG_NONFINITE = 0x2u;

// Device buffers of one stream kind (K or V), all carved from the caller's
// workspace. Units are ordered [layer][batch][kv_head] so a layer range is a
// contiguous unit range.
// Rows of D floats in each unit's fold scratch: the residual basis P
// (min(b, D) rows), later the two k+ x k+ Gram corrections (2 r^2 floats).
inline int scratch_rows(int block, int rank_k, int rank_v) {
  const int rm = rank_k > rank_v ? rank_k : rank_v;
  const int pr = block < D ? block : D;
  const int er = (2 * rm * rm + D - 1) / D;
  return pr > er ? pr : er;
}

// floats per unit of the int8 row scales: ncap rounded up to 4, so that four
// consecutive rows' scales (from a multiple of 4) are one aligned 16-byte piece
inline __host__ __device__ size_t cs_stride(int ncap) { return ((size_t)ncap + 3) & ~(size_t)3; }

struct Stream {
  void *C;          // [U][cstride] coordinates C = U Sigma (coord dtype): ncap rows of r, zero beyond column k;
                    // int8 storage keeps U = C Sigma^-1 here as codes, one scale per row in cs
  float *cs;        // [U][cs_stride(ncap)] int8 storage: scale of each stored row of U (nullptr otherwise)
  float *Bt;        // [U][r][D] basis vectors as rows, zero beyond row k
  float *sig;       // [U][r] singular values, zero beyond k
  void *ring;       // [U][rcap][D] exact window ring (kv dtype)
  float *Htop;      // [U][r][r] scratch: signed, sorted H[0:k, 0:k+] of the last fold
  float *P;         // [U][scratch_rows][D] scratch: residual basis rows, then the basis Gram correction
  float *YFP;       // [U][bmax][D] scratch: rows [F B | F P] of the last fold
  int32_t *sweeps;  // [U] core sweeps of the last fold
  float *disc;      // [U] energy dropped by the last fold
  int r;            // rank budget
  size_t cstride;   // elements of C per unit: ncap * r plus a 256-byte pad, so unit strides are
                    // not a power of two (all units stream the same offsets at once)
};

struct Layout {
  int batch, layers, kvh, qh, g;  // g = query heads per kv head
  int b, w, ncap, rcap;           // block, window, history capacity, ring capacity
  int coord_bf16, kv_bf16;
  int coord_i8;                   // int8 codes of U with per-row scales (coord_bf16 is 0 then)
  int units;                      // batch * layers * kvh
  Stream X[2];                    // 0 = K, 1 = V
  uint32_t *status;               // [16] sticky numeric flags
  // decode scratch
  uint32_t *ticket;  // [U] decode blocks finished per unit (reset to 0 by the last one)
  float *part;    // [U][nchunk_max][g][2 + rV] per-chunk (max, sum, o')
  float *wpart;   // [U][g][2 + D] window part (max, sum, o)
  int chunk;      // history rows per decode chunk
  int nchunk_max;
  // split decode partials of launches over at most split_units units
  float *spart;
  int split_units, split_max;
};

// One fold round: both stream kinds in one launch (blockIdx.y = 0 keys, 1 values).
struct FoldArgs {
  Stream X[2];
  int k[2], r[2];    // rank before the fold and rank budget, per kind
  int u0;            // first unit of the launch
  int n, b;          // history rows, block
  int rcap, head;    // ring capacity and ring index of F's first row
  int ncap, bmax;
  int pmax;          // rows of D floats per unit of the fold scratch (scratch_rows)
  uint32_t *status;
  int lds_small[2];  // float offset of the small arrays in dynamic LDS, per kind
  int mode;          // ISKV_MODE_JOINT (launch_fold) or ISKV_MODE_FIXED_COORDS (launch_core);
                     // fixed basis: launch_project
};

struct RewriteArgs {
  Stream X[2];
  int k[2], kp[2], r[2];
  int u0, n, ncap;
};

struct IngestArgs {
  const void *src[2];  // K, V rows [batch][nl_in][kvh][nrows][D]
  void *ring[2];
  int batch, kvh, nl_in, lrel0, nl;  // input layer count, first input layer of the run, layers in run
  int u0, nrows, rcap, pos;          // ring index of the first new row
};

struct DecodeArgs {
  Layout L;
  const void *q;  // [batch][nl_in][qh][D] in kv dtype
  void *out;      // [batch][nl_in][qh][D] fp32
  int nl_in, lrel0, nl, u0;
  int n, e, kK, kV, head;
  int nchunk;
  float scale;
  int wlds;  // window rows staged in LDS (set by the launcher)
  // fused append: one new K and V row per unit ([batch][nl_in][kvh][1][D]),
  // written to the ring at position e and attended as window row e
  const void *nk, *nv;
  int nnew;
  // split history (bf16 matrix-core path, nnew == 0): nsplit > 0 workgroups per
  // unit of split_rows rows each, partials [units][nsplit][g][2 + r_V + D] in spart
  int nsplit, split_rows;
  float *spart;
};

// One-shot prefill of a layer run: every unit's nrows prompt rows
struct OneshotArgs {
  Stream X[2];
  const void *src[2];  // K, V rows [batch][nl_in][kvh][nrows][D]
  int batch, kvh, nl_in, lrel0, nl;
  int u0, nrows;
  int ncap;  // history capacity (rows per unit of the int8 scale arrays)
  int gram;  // 1: R comes from the Cholesky factor of the fp64 Gram matrix (k_oneshot_gram)
  int cb;    // bytes per coordinate element (the Gram scratch sits in each unit's coordinates)
  uint32_t *status;
};

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T>
__device__ __forceinline__ float ldf(const T *p, size_t i);
template <>
__device__ __forceinline__ float ldf<float>(const float *p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ldf<uint16_t>(const uint16_t *p, size_t i) { return bf2f(p[i]); }

template <typename T>
__device__ __forceinline__ void stf(T *p, size_t i, float v);
template <>
__device__ __forceinline__ void stf<float>(float *p, size_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void stf<uint16_t>(uint16_t *p, size_t i, float v) { p[i] = f2bf(v); }

// sum over the 16 lanes of an aligned lane group
__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 8);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 1);
  return v;
}

__device__ __forceinline__ float sum64(float v) {
  v += __shfl_xor(v, 32);
  v += __shfl_xor(v, 16);
  return sum16(v);
}

// int8 storage of a row of U: scale = max|u| / 127, code = round-half-even(u * 127 / max|u|),
// the rounding decision taken in fp32 from the row's own maximum
__device__ __forceinline__ float i8_inv_step(float m) { return m > 0.f ? 127.f / m : 0.f; }
// (one rounding of v * inv to the nearest integer, ties to even, as in i8_pack4)
__device__ __forceinline__ int i8_code(float v, float inv) {
  return (int)(int8_t)(__float_as_uint(fmaf(v, inv, 12582912.0f)) & 0xffu);
}

// Four codes packed into one dword (byte i = code of v_i), each the nearest
// integer of v_i * inv, ties to even: one fma against 1.5 * 2^23 leaves that
// integer in the low mantissa bits (|v_i * inv| <= 127.5 < 2^22), whose low
// byte is the code in two's complement; two byte permutes gather them.
__device__ __forceinline__ uint32_t i8_pack4(float v0, float v1, float v2, float v3, float inv) {
  constexpr float MAGIC = 12582912.0f;
  const uint32_t a = __float_as_uint(fmaf(v0, inv, MAGIC)), b = __float_as_uint(fmaf(v1, inv, MAGIC));
  const uint32_t c = __float_as_uint(fmaf(v2, inv, MAGIC)), d = __float_as_uint(fmaf(v3, inv, MAGIC));
  return __builtin_amdgcn_perm(b, a, 0x0c0c0400u) | __builtin_amdgcn_perm(d, c, 0x04000c0cu);
}

// bf16 bits of a small integer (exact: |x| <= 256)
__device__ __forceinline__ uint32_t int_bf16(int x) { return __float_as_uint((float)x) >> 16; }

// eight int8 codes (two dwords, low byte first) as eight bf16 values packed in
// four dwords, the operand layout of the bf16 matrix-core instructions
// (each code sign-extended and converted from its byte lane in one instruction,
// exact; the upper halves of two such floats are their bf16 values)
__device__ __forceinline__ void i8x8_bf16(uint32_t w0, uint32_t w1, uint32_t out[4]) {
#pragma unroll
  for (int e = 0; e < 4; e += 2) {
    const uint32_t w = e == 0 ? w0 : w1;
    const float f0 = (float)(int8_t)w, f1 = (float)(int8_t)(w >> 8);
    const float f2 = (float)(int8_t)(w >> 16), f3 = (float)(int8_t)(w >> 24);
    out[e] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    out[e + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
  }
}

__device__ __forceinline__ float max64(float v) {
  v = fmaxf(v, __shfl_xor(v, 32));
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 8));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 1));
  return v;
}

// ---------------------------------------------------------------------------
// launchers (each returns the hipError_t of its launch)
// ---------------------------------------------------------------------------
size_t core_lds_bytes(int k, int b, int r);
hipError_t launch_core(const FoldArgs &a, int nunits, int kv_bf16, int coord_bf16, hipStream_t s);  // grid (nunits, 2)
// joint-mode fold core (k_fold.hip): grid (nunits, 2), 512 threads per unit stream
size_t fold_core_lds_bytes(int k, int b, int r);
hipError_t launch_fold(const FoldArgs &a, int nunits, int kv_bf16, int coord_bf16, hipStream_t s);
hipError_t launch_rewrite(const RewriteArgs &a, int nunits, int coord_bf16, hipStream_t s);  // K and V
// int8 storage: U <- U M in place with per-row scales, M = Sigma_old H_top Sigma_new^-1 (in Htop)
hipError_t launch_rewrite_i8(const RewriteArgs &a, int nunits, hipStream_t s);
hipError_t launch_ingest(const IngestArgs &a, int kv_bf16, hipStream_t s);
// fixed-basis fold: new rows C[n + i] = F_i B (k columns), discarded energy
hipError_t launch_project(const FoldArgs &a, int nunits, int kv_bf16, int coord_bf16, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);
// one-shot prefill: QR + Jacobi (k_oneshot_svd), then coordinates and sigma (k_oneshot_coords)
hipError_t launch_oneshot(const OneshotArgs &a, int nunits, int kv_bf16, int coord_bf16, hipStream_t s);
// one-shot coordinates and sigma on matrix cores (k_rewrite.hip): bf16 rows and
// coordinates, ranks multiples of 8
bool oneshot_coords_mfma_ok(const OneshotArgs &a, int kv_bf16, int coord_bf16);
hipError_t launch_oneshot_coords_mfma(const OneshotArgs &a, int nunits, hipStream_t s);
// int8 storage: sigma = column norms of X B^T, then U = X B^T Sigma^-1 stored per row
hipError_t launch_oneshot_coords_i8(const OneshotArgs &a, int nunits, hipStream_t s);
// true when launch_decode can take the appended row itself (nnew = 1)
bool decode_can_fuse(const DecodeArgs &a);
// true when the split (matrix-core) decode applies to these counters
bool decode_can_split(const DecodeArgs &a);
// floats of split partials per unit and split
inline size_t decode_split_floats(int g, int rank_v) { return (size_t)g * (2 + rank_v + D); }
int decode_chunk_rows(const Layout &L);  // history rows per decode block
hipError_t launch_reconstruct(const Layout &L, int which, int u, int n, int k, int e, int head,
                              float *out, hipStream_t s);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);
hipError_t launch_ring_copy(const Layout &L, int which, int u, int e, int head, void *dst,
                            const void *src, int to_ring, hipStream_t s);

}  // namespace iskv
