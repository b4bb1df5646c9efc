// Host side of the C ABI declared in include/iskv.h: configuration checks,
// workspace carve-up, per-layer counters and launch sequencing. The window
// policy follows section "Architecture Overview" of the iS-KV page (exact
// recent rows) with the fold trigger of section "Block-Incremental Decoding
// Updates" (the oldest b rows become the pending block F once the window
// holds w + b rows).
#include <new>
#include <algorithm>
#include <mutex>
#include <vector>

#include "iskv.h"
#include "iskv_internal.hpp"

using namespace iskv;

// Device memory owned by the library for iskv_decode_attn_static: the split
// decode partials of callers that cannot allocate. Each GPU the library runs
// on holds its own copy until the process ends. Host code never uses the
// symbol itself (on the host it is a stand-in, not a device address): the
// device address comes from hipGetSymbolAddress, once per device, at the
// first iskv_init on that device.
static __device__ __align__(256) unsigned char scratch[ISKV_STATIC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES];
bool g_scratch_done[MAX_DEVICES];

// device address of `scratch` on the current device (nullptr if unavailable)
void *static_scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_done[dev]) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = (e == hipSuccess) ? ptr : nullptr;
    g_scratch_done[dev] = true;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

struct iskv_ctx {
  iskv_config cfg;
  Layout L;
  void *ws;
  size_t ws_bytes;
  std::vector<int> n, e, head, kk, kv;
  bool poisoned;
  int mode;  // ISKV_MODE_*
  // caller's timing events recorded around each fold's kernels (see iskv_set_fold_events)
  hipEvent_t fev[4];
  bool fev_on;
  void *static_scratch;  // device address of `scratch` on the handle's device (or nullptr)
};

static_assert(MODE_JOINT == ISKV_MODE_JOINT && MODE_FIXED_COORDS == ISKV_MODE_FIXED_COORDS &&
                  MODE_FIXED_BASIS == ISKV_MODE_FIXED_BASIS,
              "mode values");

namespace {

constexpr size_t ALIGN = 256;
constexpr int MAX_UNITS_PER_LAUNCH = 65535;

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

bool valid_config(const iskv_config *c) {
  if (!c) return false;
  if (c->head_dim != D) return false;
  if (c->batch < 1 || c->layers < 1 || c->kv_heads < 1 || c->q_heads < 1) return false;
  if (c->q_heads % c->kv_heads != 0) return false;
  const int g = c->q_heads / c->kv_heads;
  if (g > 8) return false;
  if (c->block < 1 || c->block > D) return false;
  if (c->rank_k < 1 || c->rank_k > D || c->rank_v < 1 || c->rank_v > D) return false;
  if (c->window < 0 || c->max_tokens < 1) return false;
  if (c->coord_dtype != ISKV_F32 && c->coord_dtype != ISKV_BF16 && c->coord_dtype != ISKV_I8) return false;
  if (c->kv_dtype != ISKV_F32 && c->kv_dtype != ISKV_BF16) return false;
  if (c->coord_dtype == ISKV_I8) {
    // int8 rows run on the bf16 matrix-core kernels only: bf16 rows, ranks in
    // whole 8-column pieces, and every byte offset of a unit's rows (plus one
    // prefetch of rows) below 2^31
    if (c->kv_dtype != ISKV_BF16 || c->rank_k % 8 != 0 || c->rank_v % 8 != 0) return false;
    const long long ncap = (long long)(c->max_tokens / c->block) * c->block;
    const int rm = c->rank_k > c->rank_v ? c->rank_k : c->rank_v;
    if ((ncap + 65536) * rm >= (1LL << 31)) return false;
  }
  const long long units = (long long)c->batch * c->layers * c->kv_heads;
  if (units > (1LL << 26)) return false;
  if ((long long)c->batch * c->kv_heads > MAX_UNITS_PER_LAUNCH) return false;
  // the decode kernel keeps one score per window row and query head in LDS
  if ((long long)c->window + 2LL * c->block > 4096) return false;
  return true;
}

// Computes the layout; with base == nullptr only the size is returned.
size_t carve(const iskv_config *c, char *base, Layout *L) {
  Layout l = {};
  l.batch = c->batch;
  l.layers = c->layers;
  l.kvh = c->kv_heads;
  l.qh = c->q_heads;
  l.g = c->q_heads / c->kv_heads;
  l.b = c->block;
  l.w = c->window;
  l.ncap = (c->max_tokens / c->block) * c->block;
  l.rcap = c->window + 2 * c->block;
  l.coord_bf16 = c->coord_dtype == ISKV_BF16;
  l.coord_i8 = c->coord_dtype == ISKV_I8;
  l.kv_bf16 = c->kv_dtype == ISKV_BF16;
  l.units = c->batch * c->layers * c->kv_heads;
  l.chunk = 512 > l.rcap ? 512 : l.rcap;
  l.nchunk_max = (l.ncap + 511) / 512;  // every decode path uses >= 512 history rows per block
  if (l.nchunk_max < 1) l.nchunk_max = 1;
  const size_t U = (size_t)l.units;
  const size_t cb = l.coord_i8 ? 1 : l.coord_bf16 ? 2 : 4, kb = l.kv_bf16 ? 2 : 4;
  const int pmax = scratch_rows(c->block, c->rank_k, c->rank_v);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void * {
    void *p = base ? (void *)(base + off) : nullptr;
    off += align_up(bytes);
    return p;
  };
  for (int x = 0; x < 2; x++) {
    const int r = x == 0 ? c->rank_k : c->rank_v;
    Stream &s = l.X[x];
    s.r = r;
    // int8 rows are read in 16-byte pieces: keep every unit's rows 16-byte aligned
    s.cstride = l.coord_i8 ? ((size_t)l.ncap * r + 15) / 16 * 16 + 256 : (size_t)l.ncap * r + 256 / cb;
    s.C = take(U * s.cstride * cb);
    s.cs = l.coord_i8 ? (float *)take(U * cs_stride(l.ncap) * 4) : nullptr;
    s.Bt = (float *)take(U * r * D * 4);
    s.sig = (float *)take(U * r * 4);
    s.ring = take(U * l.rcap * D * kb);
    s.Htop = (float *)take(U * r * r * 4);
    s.P = (float *)take(U * pmax * D * 4);
    s.YFP = (float *)take(U * c->block * D * 4);
    s.sweeps = (int32_t *)take(U * 4);
    s.disc = (float *)take(U * 4);
  }
  // split decode partials: launches over at most split_units units, at most
  // split_max workgroups per unit (each split takes >= 1024 history rows)
  l.split_units = (int)(U < 128 ? U : 128);
  l.split_max = l.ncap / 1024 < 64 ? l.ncap / 1024 : 64;
  if (l.split_max < 1) l.split_max = 1;
  l.spart = (float *)take((size_t)l.split_units * l.split_max * decode_split_floats(l.g, c->rank_v) * 4);
  l.ticket = (uint32_t *)take(U * 4);
  l.part = (float *)take(U * l.nchunk_max * l.g * (2 + c->rank_v) * 4);
  l.wpart = (float *)take(U * l.g * (2 + D) * 4);
  l.status = (uint32_t *)take(64);
  if (L) *L = l;
  return off;
}

int fail_hip(iskv_t h, hipError_t e) {
  if (e != hipSuccess) {
    h->poisoned = true;
    return ISKV_ERR_HIP;
  }
  return ISKV_OK;
}

inline int unit_index(const iskv_t h, int b, int l, int hd) {
  return (l * h->L.batch + b) * h->L.kvh + hd;
}

bool same_counts(const iskv_t h, int a, int b) {
  return h->n[a] == h->n[b] && h->e[a] == h->e[b] && h->head[a] == h->head[b] &&
         h->kk[a] == h->kk[b] && h->kv[a] == h->kv[b];
}

// Largest run of layers starting at l0 (within [l0, lend)) that share counters
// and fits one launch.
int run_end(const iskv_t h, int l0, int lend) {
  const int per_layer = h->L.batch * h->L.kvh;
  int l1 = l0 + 1;
  while (l1 < lend && same_counts(h, l0, l1) && (l1 + 1 - l0) * per_layer <= MAX_UNITS_PER_LAUNCH) l1++;
  return l1;
}

inline int kplus_of(int k, int b, int r) {
  const int p = b < D - k ? b : D - k;
  const int c = k + p;
  return r < c ? r : c;
}

// Fold the oldest b window rows of layers [l0, l1) (identical counters).
int fold_run(iskv_t h, int l0, int l1, hipStream_t s) {
  const Layout &L = h->L;
  const int per_layer = L.batch * L.kvh;
  const int u0 = l0 * per_layer, nunits = (l1 - l0) * per_layer;
  const int n = h->n[l0];
  int kp[2];
  FoldArgs a = {};
  RewriteArgs ra = {};
  for (int x = 0; x < 2; x++) {
    const int k = x == 0 ? h->kk[l0] : h->kv[l0];
    kp[x] = kplus_of(k, L.b, L.X[x].r);
    a.X[x] = L.X[x];
    a.k[x] = k;
    a.r[x] = L.X[x].r;
    ra.X[x] = L.X[x];
    ra.k[x] = k;
    ra.kp[x] = kp[x];
    ra.r[x] = L.X[x].r;
  }
  a.u0 = u0;
  a.n = n;
  a.b = L.b;
  a.rcap = L.rcap;
  a.head = h->head[l0];
  a.ncap = L.ncap;
  a.bmax = L.b;
  a.pmax = scratch_rows(L.b, L.X[0].r, L.X[1].r);
  a.status = L.status;
  a.mode = h->mode;
  if (h->mode == ISKV_MODE_FIXED_BASIS && a.k[0] > 0 && a.k[1] > 0) {
    // the basis exists and is kept: store the block's projections, no core
    int rc = fail_hip(h, launch_project(a, nunits, L.kv_bf16, L.coord_bf16, s));
    if (rc) return rc;
    for (int l = l0; l < l1; l++) {
      h->n[l] += L.b;
      h->e[l] -= L.b;
      h->head[l] = (h->head[l] + L.b) % L.rcap;
    }
    return ISKV_OK;
  }
  if (a.mode == ISKV_MODE_FIXED_BASIS) a.mode = ISKV_MODE_JOINT;  // first fold builds the basis
  if (h->fev_on && fail_hip(h, hipEventRecord(h->fev[1], s))) return ISKV_ERR_HIP;
  int rc = fail_hip(h, a.mode == ISKV_MODE_JOINT ? launch_fold(a, nunits, L.kv_bf16, L.coord_bf16, s)
                                                  : launch_core(a, nunits, L.kv_bf16, L.coord_bf16, s));
  if (rc) return rc;
  if (h->fev_on && fail_hip(h, hipEventRecord(h->fev[2], s))) return ISKV_ERR_HIP;
  if (n > 0 && a.mode == ISKV_MODE_JOINT) {
    ra.u0 = u0;
    ra.n = n;
    ra.ncap = L.ncap;
    rc = fail_hip(h, L.coord_i8 ? launch_rewrite_i8(ra, nunits, s) : launch_rewrite(ra, nunits, L.coord_bf16, s));
    if (rc) return rc;
  }
  if (h->fev_on && fail_hip(h, hipEventRecord(h->fev[3], s))) return ISKV_ERR_HIP;
  for (int l = l0; l < l1; l++) {
    h->n[l] += L.b;
    h->e[l] -= L.b;
    h->head[l] = (h->head[l] + L.b) % L.rcap;
    h->kk[l] = kp[0];
    h->kv[l] = kp[1];
  }
  return ISKV_OK;
}

int ingest_run(iskv_t h, const void *k_rows, const void *v_rows, int nrows, int layer0, int nl_in,
               int l0, int l1, hipStream_t s) {
  const Layout &L = h->L;
  IngestArgs a = {};
  a.src[0] = k_rows;
  a.src[1] = v_rows;
  a.ring[0] = L.X[0].ring;
  a.ring[1] = L.X[1].ring;
  a.batch = L.batch;
  a.kvh = L.kvh;
  a.nl_in = nl_in;
  a.lrel0 = l0 - layer0;
  a.nl = l1 - l0;
  a.u0 = l0 * L.batch * L.kvh;
  a.nrows = nrows;
  a.rcap = L.rcap;
  a.pos = (h->head[l0] + h->e[l0]) % L.rcap;
  return fail_hip(h, launch_ingest(a, L.kv_bf16, s));
}

bool bad_layers(const iskv_t h, int layer0, int nlayers) {
  return layer0 < 0 || nlayers < 1 || layer0 + nlayers > h->L.layers;
}

bool bad_unit(const iskv_t h, int which, int b, int l, int hd) {
  return (which != 0 && which != 1) || b < 0 || b >= h->L.batch || l < 0 || l >= h->L.layers ||
         hd < 0 || hd >= h->L.kvh;
}

}  // namespace

extern "C" {

size_t iskv_workspace_bytes(const iskv_config *cfg) {
  if (!valid_config(cfg)) return 0;
  return carve(cfg, nullptr, nullptr);
}

int iskv_init(const iskv_config *cfg, void *dev_ws, size_t ws_bytes, void *stream, iskv_t *out) {
  if (!out) return ISKV_ERR_ARG;
  *out = nullptr;
  if (!valid_config(cfg)) return ISKV_ERR_ARG;
  const size_t need = carve(cfg, nullptr, nullptr);
  if (!dev_ws || ws_bytes < need || ((uintptr_t)dev_ws % ALIGN) != 0) return ISKV_ERR_WORKSPACE;
  iskv_ctx *h = new (std::nothrow) iskv_ctx();
  if (!h) return ISKV_ERR_ARG;
  h->cfg = *cfg;
  carve(cfg, (char *)dev_ws, &h->L);
  h->ws = dev_ws;
  h->ws_bytes = ws_bytes;
  h->n.assign(cfg->layers, 0);
  h->e.assign(cfg->layers, 0);
  h->head.assign(cfg->layers, 0);
  h->kk.assign(cfg->layers, 0);
  h->kv.assign(cfg->layers, 0);
  h->poisoned = false;
  h->mode = ISKV_MODE_JOINT;
  h->fev_on = false;
  h->static_scratch = static_scratch_for_current_device();
  if (launch_zero(dev_ws, need, (hipStream_t)stream) != hipSuccess) {
    delete h;
    return ISKV_ERR_HIP;
  }
  *out = h;
  return ISKV_OK;
}

int iskv_reset(iskv_t h, void *stream) {
  if (!h) return ISKV_ERR_ARG;
  if (h->poisoned) return ISKV_ERR_POISONED;
  for (int l = 0; l < h->L.layers; l++) h->n[l] = h->e[l] = h->head[l] = h->kk[l] = h->kv[l] = 0;
  return fail_hip(h, launch_zero(h->L.status, 64, (hipStream_t)stream));
}

int iskv_set_fold_events(iskv_t h, void *const *events) {
  if (!h) return ISKV_ERR_ARG;
  if (!events) {
    h->fev_on = false;
    return ISKV_OK;
  }
  for (int i = 0; i < 4; i++)
    if (!events[i]) return ISKV_ERR_ARG;
  for (int i = 0; i < 4; i++) h->fev[i] = (hipEvent_t)events[i];
  h->fev_on = true;
  return ISKV_OK;
}

int iskv_set_mode(iskv_t h, int32_t mode) {
  if (!h) return ISKV_ERR_ARG;
  if (mode != ISKV_MODE_JOINT && mode != ISKV_MODE_FIXED_COORDS && mode != ISKV_MODE_FIXED_BASIS)
    return ISKV_ERR_ARG;
  if (h->L.coord_i8 && mode != ISKV_MODE_JOINT) return ISKV_ERR_ARG;  // int8 storage: joint update only
  h->mode = mode;
  return ISKV_OK;
}

int iskv_append_block(iskv_t h, const void *k_rows, const void *v_rows, int32_t nrows, int32_t layer0,
                      int32_t nlayers, void *stream) {
  if (!h || !k_rows || !v_rows) return ISKV_ERR_ARG;
  if (h->poisoned) return ISKV_ERR_POISONED;
  if (bad_layers(h, layer0, nlayers) || nrows < 1 || nrows > h->L.b) return ISKV_ERR_ARG;
  const int w = h->L.w, b = h->L.b;
  for (int l = layer0; l < layer0 + nlayers; l++) {
    const int e2 = h->e[l] + nrows;
    if ((long long)h->n[l] + e2 > h->cfg.max_tokens) return ISKV_ERR_CAPACITY;
    if (e2 >= w + b && h->n[l] + b > h->L.ncap) return ISKV_ERR_CAPACITY;
  }
  hipStream_t s = (hipStream_t)stream;
  for (int l0 = layer0; l0 < layer0 + nlayers;) {
    const int l1 = run_end(h, l0, layer0 + nlayers);
    if (h->fev_on && h->e[l0] + nrows >= w + b && fail_hip(h, hipEventRecord(h->fev[0], s)))
      return ISKV_ERR_HIP;
    int rc = ingest_run(h, k_rows, v_rows, nrows, layer0, nlayers, l0, l1, s);
    if (rc) return rc;
    for (int l = l0; l < l1; l++) h->e[l] += nrows;
    if (h->e[l0] >= w + b) {
      rc = fold_run(h, l0, l1, s);
      if (rc) return rc;
    }
    l0 = l1;
  }
  return ISKV_OK;
}

int iskv_prefill_block(iskv_t h, const void *k_rows, const void *v_rows, int32_t layer0, int32_t nlayers,
                       void *stream) {
  if (!h || !k_rows || !v_rows) return ISKV_ERR_ARG;
  if (h->poisoned) return ISKV_ERR_POISONED;
  if (bad_layers(h, layer0, nlayers)) return ISKV_ERR_ARG;
  const int b = h->L.b;
  for (int l = layer0; l < layer0 + nlayers; l++) {
    if (h->e[l] != 0) return ISKV_ERR_STATE;
    if ((long long)h->n[l] + b > h->cfg.max_tokens || h->n[l] + b > h->L.ncap) return ISKV_ERR_CAPACITY;
  }
  hipStream_t s = (hipStream_t)stream;
  for (int l0 = layer0; l0 < layer0 + nlayers;) {
    const int l1 = run_end(h, l0, layer0 + nlayers);
    int rc = ingest_run(h, k_rows, v_rows, b, layer0, nlayers, l0, l1, s);
    if (rc) return rc;
    for (int l = l0; l < l1; l++) h->e[l] += b;
    rc = fold_run(h, l0, l1, s);
    if (rc) return rc;
    l0 = l1;
  }
  return ISKV_OK;
}

int iskv_prefill_oneshot(iskv_t h, const void *k_rows, const void *v_rows, int32_t nrows, int32_t layer0,
                         int32_t nlayers, void *stream) {
  if (!h || !k_rows || !v_rows) return ISKV_ERR_ARG;
  if (h->poisoned) return ISKV_ERR_POISONED;
  if (bad_layers(h, layer0, nlayers) || nrows < 1) return ISKV_ERR_ARG;
  for (int l = layer0; l < layer0 + nlayers; l++) {
    if (h->n[l] != 0 || h->e[l] != 0) return ISKV_ERR_STATE;
    if ((long long)nrows > h->cfg.max_tokens || nrows > h->L.ncap) return ISKV_ERR_CAPACITY;
  }
  const Layout &L = h->L;
  hipStream_t s = (hipStream_t)stream;
  const int per_layer = L.batch * L.kvh;
  for (int l0 = layer0; l0 < layer0 + nlayers;) {
    const int l1 = run_end(h, l0, layer0 + nlayers);
    OneshotArgs a = {};
    for (int x = 0; x < 2; x++) a.X[x] = L.X[x];
    a.src[0] = k_rows;
    a.src[1] = v_rows;
    a.batch = L.batch;
    a.kvh = L.kvh;
    a.nl_in = nlayers;
    a.lrel0 = l0 - layer0;
    a.nl = l1 - l0;
    a.u0 = l0 * per_layer;
    a.nrows = nrows;
    a.ncap = L.ncap;
    a.status = L.status;
    int rc = fail_hip(h, launch_oneshot(a, (l1 - l0) * per_layer, L.kv_bf16, L.coord_bf16, s));
    if (rc) return rc;
    for (int l = l0; l < l1; l++) {
      h->n[l] = nrows;
      h->e[l] = 0;
      h->head[l] = 0;
      h->kk[l] = std::min(std::min(L.X[0].r, (int)nrows), D);
      h->kv[l] = std::min(std::min(L.X[1].r, (int)nrows), D);
    }
    l0 = l1;
  }
  return ISKV_OK;
}

// Split the history of each unit over several workgroups when a launch has
// too few units to fill the chip (e.g. one layer per call): at most smax
// splits of >= 1024 rows (multiples of 32), about 512 workgroups in all.
static void choose_split(DecodeArgs &a, int nunits, int smax, float *spart, bool force) {
  a.nsplit = 0;
  if (!decode_can_split(a)) return;
  int ns = 1;
  if (2 * nunits <= 256 && a.n >= 2048) {
    ns = (512 + nunits - 1) / nunits;
    if (ns > smax) ns = smax;
    if (ns > a.n / 1024) ns = a.n / 1024;
    if (ns < 1) ns = 1;
  }
  if (ns < 2 && !force) return;
  int rows = (a.n + ns - 1) / ns;
  rows = ((rows + 31) / 32) * 32;
  if (rows < 32) rows = 32;
  a.split_rows = rows;
  a.nsplit = (a.n + rows - 1) / rows;
  if (a.nsplit < 1) a.nsplit = 1;
  a.spart = spart;
}

static DecodeArgs decode_args(iskv_t h, const void *q, float *out, int layer0, int nlayers, int l0, int l1,
                              float scale) {
  DecodeArgs a = {};
  a.L = h->L;
  a.q = q;
  a.out = out;
  a.nl_in = nlayers;
  a.lrel0 = l0 - layer0;
  a.nl = l1 - l0;
  a.u0 = l0 * h->L.batch * h->L.kvh;
  a.n = h->n[l0];
  a.e = h->e[l0];
  a.kK = h->kk[l0];
  a.kV = h->kv[l0];
  a.head = h->head[l0];
  const int chunk = decode_chunk_rows(h->L);
  a.nchunk = (a.n + chunk - 1) / chunk;
  a.scale = scale;
  const int nunits = h->L.batch * (l1 - l0) * h->L.kvh;
  if (nunits <= h->L.split_units) choose_split(a, nunits, h->L.split_max, h->L.spart, false);
  return a;
}

int iskv_decode_attn(iskv_t h, const void *q, float *out, int32_t layer0, int32_t nlayers, float scale,
                     void *stream) {
  if (!h || !q || !out) return ISKV_ERR_ARG;
  if (h->poisoned) return ISKV_ERR_POISONED;
  if (bad_layers(h, layer0, nlayers)) return ISKV_ERR_ARG;
  for (int l = layer0; l < layer0 + nlayers; l++)
    if (h->n[l] + h->e[l] == 0) return ISKV_ERR_STATE;
  hipStream_t s = (hipStream_t)stream;
  for (int l0 = layer0; l0 < layer0 + nlayers;) {
    const int l1 = run_end(h, l0, layer0 + nlayers);
    const DecodeArgs a = decode_args(h, q, out, layer0, nlayers, l0, l1, scale);
    int rc = fail_hip(h, launch_decode(a, s));
    if (rc) return rc;
    l0 = l1;
  }
  return ISKV_OK;
}

int iskv_decode_attn_static(iskv_t h, const void *q, float *out, int32_t layer0, int32_t nlayers, float scale,
                            void *stream) {
  if (!h || !q || !out) return ISKV_ERR_ARG;
  if (h->poisoned) return ISKV_ERR_POISONED;
  if (bad_layers(h, layer0, nlayers)) return ISKV_ERR_ARG;
  for (int l = layer0; l < layer0 + nlayers; l++)
    if (h->n[l] + h->e[l] == 0) return ISKV_ERR_STATE;
  if (!h->static_scratch) return ISKV_ERR_HIP;
  // every launch is planned (and checked against the array) before any is enqueued
  std::vector<DecodeArgs> plan;
  for (int l0 = layer0; l0 < layer0 + nlayers;) {
    const int l1 = run_end(h, l0, layer0 + nlayers);
    DecodeArgs a = decode_args(h, q, out, layer0, nlayers, l0, l1, scale);
    if (!decode_can_split(a)) return ISKV_ERR_ARG;
    const int nunits = h->L.batch * (l1 - l0) * h->L.kvh;
    const size_t per = decode_split_floats(h->L.g, h->L.X[1].r) * sizeof(float);
    choose_split(a, nunits, 64, (float *)h->static_scratch, true);
    if ((size_t)nunits * a.nsplit * per > ISKV_STATIC_SCRATCH_BYTES) {
      a.nsplit = 0;
      choose_split(a, 1 << 20, 1, (float *)h->static_scratch, true);  // one partial per unit
      if ((size_t)nunits * a.nsplit * per > ISKV_STATIC_SCRATCH_BYTES) return ISKV_ERR_SCRATCH;
    }
    plan.push_back(a);
    l0 = l1;
  }
  hipStream_t s = (hipStream_t)stream;
  for (const DecodeArgs &a : plan) {
    const int rc = fail_hip(h, launch_decode(a, s));
    if (rc) return rc;
  }
  return ISKV_OK;
}

int iskv_append_decode(iskv_t h, const void *k_rows, const void *v_rows, const void *q, float *out,
                       int32_t layer0, int32_t nlayers, float scale, void *stream) {
  if (!h || !k_rows || !v_rows || !q || !out) return ISKV_ERR_ARG;
  if (h->poisoned) return ISKV_ERR_POISONED;
  if (bad_layers(h, layer0, nlayers)) return ISKV_ERR_ARG;
  const int w = h->L.w, b = h->L.b;
  bool fuse = true;
  for (int l = layer0; l < layer0 + nlayers; l++) {
    const int e2 = h->e[l] + 1;
    if ((long long)h->n[l] + e2 > h->cfg.max_tokens) return ISKV_ERR_CAPACITY;
    if (e2 >= w + b && h->n[l] + b > h->L.ncap) return ISKV_ERR_CAPACITY;
    if (e2 >= w + b) fuse = false;  // this append folds: ingest, fold, then decode
  }
  for (int l0 = layer0; fuse && l0 < layer0 + nlayers;) {
    const int l1 = run_end(h, l0, layer0 + nlayers);
    DecodeArgs a = decode_args(h, q, out, layer0, nlayers, l0, l1, scale);
    a.nk = k_rows;
    a.nv = v_rows;
    fuse = decode_can_fuse(a);
    l0 = l1;
  }
  if (!fuse) {
    const int rc = iskv_append_block(h, k_rows, v_rows, 1, layer0, nlayers, stream);
    if (rc) return rc;
    return iskv_decode_attn(h, q, out, layer0, nlayers, scale, stream);
  }
  hipStream_t s = (hipStream_t)stream;
  for (int l0 = layer0; l0 < layer0 + nlayers;) {
    const int l1 = run_end(h, l0, layer0 + nlayers);
    DecodeArgs a = decode_args(h, q, out, layer0, nlayers, l0, l1, scale);
    a.nk = k_rows;
    a.nv = v_rows;
    a.nnew = 1;
    a.nsplit = 0;  // the fused append runs one workgroup per unit
    const int rc = fail_hip(h, launch_decode(a, s));
    if (rc) return rc;
    for (int l = l0; l < l1; l++) h->e[l] += 1;
    l0 = l1;
  }
  return ISKV_OK;
}

int iskv_reconstruct(iskv_t h, int32_t which, int32_t b, int32_t layer, int32_t head, float *dev_out,
                     void *stream) {
  if (!h || !dev_out) return ISKV_ERR_ARG;
  if (h->poisoned) return ISKV_ERR_POISONED;
  if (bad_unit(h, which, b, layer, head)) return ISKV_ERR_ARG;
  const int u = unit_index(h, b, layer, head);
  const int k = which == 0 ? h->kk[layer] : h->kv[layer];
  return fail_hip(h, launch_reconstruct(h->L, which, u, h->n[layer], k, h->e[layer], h->head[layer],
                                        dev_out, (hipStream_t)stream));
}

int iskv_counts(iskv_t h, int32_t layer, int32_t *n, int32_t *e, int32_t *k_k, int32_t *k_v) {
  if (!h || layer < 0 || layer >= h->L.layers) return ISKV_ERR_ARG;
  if (n) *n = h->n[layer];
  if (e) *e = h->e[layer];
  if (k_k) *k_k = h->kk[layer];
  if (k_v) *k_v = h->kv[layer];
  return ISKV_OK;
}

int iskv_export_state(iskv_t h, int32_t which, int32_t b, int32_t layer, int32_t head, void *C,
                      float *sigma, float *Bt, void *window, void *stream) {
  if (!h) return ISKV_ERR_ARG;
  if (h->poisoned) return ISKV_ERR_POISONED;
  if (bad_unit(h, which, b, layer, head)) return ISKV_ERR_ARG;
  const Layout &L = h->L;
  const Stream &X = L.X[which];
  const int u = unit_index(h, b, layer, head);
  hipStream_t s = (hipStream_t)stream;
  const size_t cb = L.coord_i8 ? 1 : L.coord_bf16 ? 2 : 4;
  if (C && h->n[layer] > 0) {
    const char *src = (const char *)X.C + (size_t)u * X.cstride * cb;
    if (fail_hip(h, hipMemcpyAsync(C, src, (size_t)h->n[layer] * X.r * cb, hipMemcpyDeviceToDevice, s)))
      return ISKV_ERR_HIP;
  }
  if (sigma &&
      fail_hip(h, hipMemcpyAsync(sigma, X.sig + (size_t)u * X.r, X.r * 4, hipMemcpyDeviceToDevice, s)))
    return ISKV_ERR_HIP;
  if (Bt &&
      fail_hip(h, hipMemcpyAsync(Bt, X.Bt + (size_t)u * X.r * D, (size_t)X.r * D * 4, hipMemcpyDeviceToDevice, s)))
    return ISKV_ERR_HIP;
  if (window && fail_hip(h, launch_ring_copy(L, which, u, h->e[layer], h->head[layer], window, nullptr, 0, s)))
    return ISKV_ERR_HIP;
  return ISKV_OK;
}

int iskv_set_counts(iskv_t h, int32_t layer, int32_t n, int32_t e, int32_t k_k, int32_t k_v) {
  if (!h || layer < 0 || layer >= h->L.layers) return ISKV_ERR_ARG;
  if (h->poisoned) return ISKV_ERR_POISONED;
  const int b = h->L.b;
  auto kmax = [&](int r) { int m = r < n ? r : n; return m < D ? m : D; };
  if (n < 0 || n > h->L.ncap || e < 0 || e >= h->L.w + b) return ISKV_ERR_ARG;
  if ((long long)n + e > h->cfg.max_tokens) return ISKV_ERR_CAPACITY;
  if (k_k < 0 || k_k > kmax(h->L.X[0].r) || k_v < 0 || k_v > kmax(h->L.X[1].r)) return ISKV_ERR_ARG;
  if ((n > 0) != (k_k > 0) || (n > 0) != (k_v > 0)) return ISKV_ERR_ARG;
  h->n[layer] = n;
  h->e[layer] = e;
  h->head[layer] = 0;
  h->kk[layer] = k_k;
  h->kv[layer] = k_v;
  return ISKV_OK;
}

int iskv_import_state(iskv_t h, int32_t which, int32_t b, int32_t layer, int32_t head, const void *C,
                      const float *sigma, const float *Bt, const void *window, void *stream) {
  if (!h) return ISKV_ERR_ARG;
  if (h->poisoned) return ISKV_ERR_POISONED;
  if (bad_unit(h, which, b, layer, head)) return ISKV_ERR_ARG;
  const Layout &L = h->L;
  const Stream &X = L.X[which];
  const int u = unit_index(h, b, layer, head);
  hipStream_t s = (hipStream_t)stream;
  const size_t cb = L.coord_i8 ? 1 : L.coord_bf16 ? 2 : 4;
  if (C && h->n[layer] > 0) {
    char *dst = (char *)X.C + (size_t)u * X.cstride * cb;
    if (fail_hip(h, hipMemcpyAsync(dst, C, (size_t)h->n[layer] * X.r * cb, hipMemcpyDeviceToDevice, s)))
      return ISKV_ERR_HIP;
  }
  if (sigma &&
      fail_hip(h, hipMemcpyAsync(X.sig + (size_t)u * X.r, sigma, X.r * 4, hipMemcpyDeviceToDevice, s)))
    return ISKV_ERR_HIP;
  if (Bt &&
      fail_hip(h, hipMemcpyAsync(X.Bt + (size_t)u * X.r * D, Bt, (size_t)X.r * D * 4, hipMemcpyDeviceToDevice, s)))
    return ISKV_ERR_HIP;
  if (window && fail_hip(h, launch_ring_copy(L, which, u, h->e[layer], h->head[layer], nullptr, window, 1, s)))
    return ISKV_ERR_HIP;
  return ISKV_OK;
}

static int copy_scales(iskv_t h, int which, int b, int layer, int head, float *out, const float *in,
                       void *stream) {
  if (!h || (!out && !in)) return ISKV_ERR_ARG;
  if (h->poisoned) return ISKV_ERR_POISONED;
  if (bad_unit(h, which, b, layer, head) || !h->L.coord_i8) return ISKV_ERR_ARG;
  const Stream &X = h->L.X[which];
  float *sc = X.cs + (size_t)unit_index(h, b, layer, head) * cs_stride(h->L.ncap);
  const size_t bytes = (size_t)h->n[layer] * 4;
  if (bytes == 0) return ISKV_OK;
  return fail_hip(h, out ? hipMemcpyAsync(out, sc, bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream)
                         : hipMemcpyAsync(sc, in, bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream));
}

int iskv_export_scales(iskv_t h, int32_t which, int32_t b, int32_t layer, int32_t head, float *scales,
                       void *stream) {
  if (!scales) return ISKV_ERR_ARG;
  return copy_scales(h, which, b, layer, head, scales, nullptr, stream);
}

int iskv_import_scales(iskv_t h, int32_t which, int32_t b, int32_t layer, int32_t head, const float *scales,
                       void *stream) {
  if (!scales) return ISKV_ERR_ARG;
  return copy_scales(h, which, b, layer, head, nullptr, scales, stream);
}

int iskv_fold_stats(iskv_t h, int32_t which, int32_t *sweeps, float *discarded, void *stream) {
  if (!h || (which != 0 && which != 1)) return ISKV_ERR_ARG;
  if (h->poisoned) return ISKV_ERR_POISONED;
  const Stream &X = h->L.X[which];
  hipStream_t s = (hipStream_t)stream;
  const size_t bytes = (size_t)h->L.units * 4;
  if (sweeps && fail_hip(h, hipMemcpyAsync(sweeps, X.sweeps, bytes, hipMemcpyDeviceToDevice, s)))
    return ISKV_ERR_HIP;
  if (discarded && fail_hip(h, hipMemcpyAsync(discarded, X.disc, bytes, hipMemcpyDeviceToDevice, s)))
    return ISKV_ERR_HIP;
  return ISKV_OK;
}

int iskv_status(iskv_t h, void *stream, uint32_t *flags) {
  if (!h || !flags) return ISKV_ERR_ARG;
  if (h->poisoned) return ISKV_ERR_POISONED;
  hipStream_t s = (hipStream_t)stream;
  uint32_t f = 0;
  if (fail_hip(h, hipStreamSynchronize(s))) return ISKV_ERR_HIP;
  if (fail_hip(h, hipMemcpy(&f, h->L.status, 4, hipMemcpyDeviceToHost))) return ISKV_ERR_HIP;
  *flags = f;
  return f ? ISKV_ERR_NUMERIC : ISKV_OK;
}

int iskv_destroy(iskv_t h) {
  if (!h) return ISKV_ERR_ARG;
  delete h;
  return ISKV_OK;
}

const char *iskv_strerror(int code) {
  switch (code) {
    case ISKV_OK: return "ok";
    case ISKV_ERR_ARG: return "invalid argument";
    case ISKV_ERR_WORKSPACE: return "workspace too small or misaligned";
    case ISKV_ERR_CAPACITY: return "token capacity exceeded";
    case ISKV_ERR_HIP: return "HIP runtime error";
    case ISKV_ERR_NUMERIC: return "numeric flag set (sweep cap or non-finite value)";
    case ISKV_ERR_POISONED: return "handle poisoned by an earlier launch failure";
    case ISKV_ERR_STATE: return "call not valid in the current cache state";
    case ISKV_ERR_SCRATCH: return "call needs more than the library's static scratch array";
    default: return "unknown status";
  }
}

}  // extern "C"
