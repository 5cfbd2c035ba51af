// C ABI of the sink-attention library: argument validation, the host-side
// KV cache handle with snapshot bookkeeping, the YaRN rate table, and the
// kernel launches.  Every entry point validates everything before it
// enqueues anything; on a non-OK status no work is queued and no state
// changes.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>
#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/sinkattn.h"
#include "sa_kernels.h"
#include "sa_sample.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return SA_OK;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int elt_bytes(int dtype) { return dtype == SA_BF16 ? 2 : (dtype == SA_F32 ? 4 : 0); }

int hip_fail(hipError_t e, const char* what) {
  return fail(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// "MoE-Xtend" README, ROPE + SCALING: blended inverse frequencies.
int yarn_table(const sa_yarn* y, int d_h, double* inv, double* conc) {
  if (!y) return fail(SA_ERR_ARG, "yarn parameters are null");
  if (y->d_h != d_h) return fail(SA_ERR_SHAPE, "yarn d_h %d != d_h %d", y->d_h, d_h);
  if (d_h <= 0 || (d_h & 1)) return fail(SA_ERR_ARG, "d_h must be even and positive");
  if (!(y->base > 1.0) || !(y->factor >= 1.0) || !(y->ntk_alpha > 0.0) ||
      !(y->ntk_beta > y->ntk_alpha) || y->orig_ctx <= 0)
    return fail(SA_ERR_ARG, "yarn needs base > 1, factor >= 1, 0 < alpha < beta, orig_ctx > 0");
  const int half = d_h / 2;
  const double L = (double)y->orig_ctx;
  const double two_pi = 2.0 * M_PI;
  // cutpoints in pair-index space: where L * theta_i / (2 pi) == beta, alpha
  const double i_beta = half * std::log(L / (y->ntk_beta * two_pi)) / std::log(y->base);
  const double i_alpha = half * std::log(L / (y->ntk_alpha * two_pi)) / std::log(y->base);
  for (int i = 0; i < half; ++i) {
    const double f = std::pow(y->base, (double)i / (double)half);
    const double extra = 1.0 / f;
    const double inter = 1.0 / (y->factor * f);
    double ramp = ((double)i - i_beta) / (i_alpha - i_beta);
    ramp = ramp < 0.0 ? 0.0 : (ramp > 1.0 ? 1.0 : ramp);
    const double keep = 1.0 - ramp;                 // 1 on fast pairs
    inv[i] = inter * (1.0 - keep) + extra * keep;
  }
  *conc = 0.1 * std::log(y->factor) + 1.0;
  return SA_OK;
}

std::atomic<uint64_t> g_next_id{1};

}  // namespace

// Decode partials of sinkattn_decode_noalloc: a static device array (each
// GPU the library runs on holds its own copy until the process ends).  On
// the host `scratch` names a stand-in, not a device address: its address on
// a device comes from hipGetSymbolAddress, asked once per device with that
// device current, and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[SA_DECODE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address in *out when `need` bytes fit;
// SA_ERR_ARG (nothing touched) when they do not.
int static_scratch(size_t need, void** out) {
  if (need > (size_t)SA_DECODE_SCRATCH_BYTES)
    return fail(SA_ERR_ARG,
                "decode needs %zu bytes of partials, the static scratch holds %zu: use "
                "sinkattn_decode with a workspace", need, (size_t)SA_DECODE_SCRATCH_BYTES);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SA_ERR_ARG, "device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(SA_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SA_OK;
}
}  // namespace

// Offsets, high-water marks and rewrite records are global positions.  A
// linear cache holds position p in row p - base (base is 0 unless the cache
// was filled by kv_ring_stage); a ring holds p in row p mod capacity.
struct sa_kv_cache {
  void* k;
  void* v;
  int dtype;
  int B, n_kv, d_h;
  int64_t capacity;
  int64_t offset;
  int64_t base;
  bool ring;
  uint64_t id;
  uint64_t stamp;
  // (stamp, first position) of appends that began below the high-water
  // mark, i.e. that may have overwritten rows some snapshot relies on.
  std::vector<std::pair<uint64_t, int64_t>> rewrites;
  int64_t high_water;
  // a stage cache: the ring it was staged from and that ring's stamp then
  uint64_t staged_from;
  uint64_t staged_stamp;
};

extern "C" {

const char* sa_last_error(void) { return g_err.c_str(); }

int sa_yarn_inv_freq(const sa_yarn* y, double* inv_freq, double* concentration) {
  if (!y || !inv_freq || !concentration) return fail(SA_ERR_ARG, "null argument");
  if (y->d_h > 2 * SA_MAX_HALF) return fail(SA_ERR_SHAPE, "d_h > %d", 2 * SA_MAX_HALF);
  int st = yarn_table(y, y->d_h, inv_freq, concentration);
  return st == SA_OK ? ok() : st;
}

int64_t sa_kv_cache_bytes(int64_t L, int64_t B, int64_t T, int64_t H_kv, int64_t d,
                          int64_t dtype_bytes) {
  if (L < 0 || B < 0 || T < 0 || H_kv < 0 || d < 0 || dtype_bytes < 0) return -1;
  int64_t f[6] = {2, L, B, T, H_kv, d};
  int64_t r = dtype_bytes;
  for (int i = 0; i < 6; ++i) {
    if (f[i] != 0 && r > INT64_MAX / f[i]) return -1;
    r *= f[i];
  }
  return r;
}

int yarn_rope(const void* x, void* y, int dtype, int B, int T, int n_heads, int d_h,
              int64_t offset, const sa_yarn* yarn, void* stream) {
  if (!x || !y) return fail(SA_ERR_ARG, "x or y is null");
  if (misaligned(x) || misaligned(y)) return fail(SA_ERR_ARG, "x and y must be 16-byte aligned");
  const int eb = elt_bytes(dtype);
  if (!eb) return fail(SA_ERR_DTYPE, "unknown dtype %d", dtype);
  if (B <= 0 || T < 0 || n_heads <= 0 || offset < 0)
    return fail(SA_ERR_ARG, "need B > 0, T >= 0, n_heads > 0, offset >= 0");
  if (d_h <= 0 || d_h % 8 || d_h > 2 * SA_MAX_HALF)
    return fail(SA_ERR_SHAPE, "d_h must be a positive multiple of 8 up to %d", 2 * SA_MAX_HALF);
  if ((int64_t)B * T > INT32_MAX) return fail(SA_ERR_ARG, "B*T too large");
  const char* xb = static_cast<const char*>(x);
  const char* yb = static_cast<const char*>(y);
  const int64_t bytes = (int64_t)B * T * n_heads * d_h * eb;
  if (xb != yb && xb < yb + bytes && yb < xb + bytes)
    return fail(SA_ERR_ARG, "x and y overlap without being the same buffer");
  RopeArgs a;
  memset(&a, 0, sizeof a);
  int st = yarn_table(yarn, d_h, a.inv_freq, &a.conc);
  if (st != SA_OK) return st;
  if (T == 0) return ok();
  a.src = x;
  a.x = y;
  a.offset = offset;
  a.BT = B * T;
  a.T = T;
  a.H = n_heads;
  a.d = d_h;
  hipError_t e = launch_rope(a, eb, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "rope launch");
  return ok();
}

int yarn_rope_apply(void* x, int dtype, int B, int T, int n_heads, int d_h, int64_t offset,
                    const sa_yarn* y, void* stream) {
  return yarn_rope(x, x, dtype, B, T, n_heads, d_h, offset, y, stream);
}

namespace {
static int cache_new(sa_kv_cache** out, void* k, void* v, int dtype, int B, int64_t capacity, int n_kv,
              int d_h, int64_t offset, bool ring) {
  if (!out || !k || !v) return fail(SA_ERR_ARG, "null argument");
  if (misaligned(k) || misaligned(v)) return fail(SA_ERR_ARG, "k and v must be 16-byte aligned");
  if (!elt_bytes(dtype)) return fail(SA_ERR_DTYPE, "unknown dtype %d", dtype);
  if (B <= 0 || n_kv <= 0 || d_h <= 0) return fail(SA_ERR_ARG, "need B, n_kv, d_h > 0");
  if (capacity <= 0 || capacity % 32)
    return fail(SA_ERR_SHAPE, "capacity must be a positive multiple of 32 (got %lld)",
                (long long)capacity);
  if (d_h % 8 || d_h > 2 * SA_MAX_HALF)
    return fail(SA_ERR_SHAPE, "d_h must be a multiple of 8 up to %d", 2 * SA_MAX_HALF);
  if (offset < 0 || offset > capacity)
    return fail(SA_ERR_CAPACITY, "initial offset %lld outside [0, capacity]", (long long)offset);
  sa_kv_cache* c = new (std::nothrow) sa_kv_cache();
  if (!c) return fail(SA_ERR_ARG, "out of host memory");
  c->k = k;
  c->v = v;
  c->dtype = dtype;
  c->B = B;
  c->n_kv = n_kv;
  c->d_h = d_h;
  c->capacity = capacity;
  c->offset = offset;
  c->base = 0;
  c->ring = ring;
  c->high_water = offset;
  c->id = g_next_id.fetch_add(1);
  c->stamp = 0;
  c->staged_from = 0;
  c->staged_stamp = 0;
  *out = c;
  return ok();
}
}  // namespace

int kv_cache_create(sa_kv_cache** out, void* k, void* v, int dtype, int B, int64_t capacity,
                    int n_kv, int d_h, int64_t offset) {
  return cache_new(out, k, v, dtype, B, capacity, n_kv, d_h, offset, false);
}

int kv_cache_init(sa_kv_cache** out, void* k, void* v, int dtype, int B, int64_t capacity,
                  int n_kv, int d_h, int64_t offset) {
  return kv_cache_create(out, k, v, dtype, B, capacity, n_kv, d_h, offset);
}

int kv_ring_create(sa_kv_cache** out, void* k, void* v, int dtype, int B, int window, int n_kv,
                   int d_h) {
  if (window <= 0 || window % 32)
    return fail(SA_ERR_SHAPE, "a ring's window must be a positive multiple of 32 (got %d)", window);
  return cache_new(out, k, v, dtype, B, window, n_kv, d_h, 0, true);
}

int kv_cache_destroy(sa_kv_cache* c) {
  if (!c) return fail(SA_ERR_ARG, "null cache");
  delete c;
  return ok();
}

int64_t kv_cache_offset(const sa_kv_cache* c) { return c ? c->offset : -1; }

int64_t kv_cache_base(const sa_kv_cache* c) {
  if (!c) return -1;
  if (c->ring) return c->offset > c->capacity ? c->offset - c->capacity : 0;
  return c->base;
}

namespace {
// Launch plan of an append: one run of cache rows, or two for a ring whose
// rows wrap past its end.  Source rows [0, t0) are not written: a ring of W
// rows keeps only the last W rows of a longer append.
struct AppendPlan {
  AppendArgs seg[2];
  int nseg;
  int t0;
};
// Checks shared by the append entry points; fills the plan.
static int append_plan(sa_kv_cache* c, const void* k, const void* v, int T_new, AppendPlan* pl) {
  if (!c || !k || !v) return fail(SA_ERR_ARG, "null argument");
  if (misaligned(k) || misaligned(v)) return fail(SA_ERR_ARG, "k and v must be 16-byte aligned");
  if (T_new <= 0) return fail(SA_ERR_ARG, "T_new must be positive");
  AppendArgs a;
  memset(&a, 0, sizeof a);
  a.k_src = k;
  a.v_src = v;
  a.kc = c->k;
  a.vc = c->v;
  a.B = c->B;
  a.n_kv = c->n_kv;
  a.d = c->d_h;
  a.C = c->capacity;
  a.src_T = T_new;
  if (!c->ring) {
    const int64_t row = c->offset - c->base;
    if (row + T_new > c->capacity)
      return fail(SA_ERR_CAPACITY, "append of %d rows at row %lld exceeds capacity %lld", T_new,
                  (long long)row, (long long)c->capacity);
    a.T_new = T_new;
    a.o = row;
    a.src_t0 = 0;
    a.pos0 = c->offset;
    pl->seg[0] = a;
    pl->nseg = 1;
    pl->t0 = 0;
    return SA_OK;
  }
  const int64_t W = c->capacity;
  const int t0 = T_new > W ? (int)(T_new - W) : 0;
  const int n = T_new - t0;
  const int64_t p = c->offset + t0;                  // position of the first kept row
  const int64_t s0 = p % W;
  const int n1 = (int)std::min<int64_t>(n, W - s0);
  a.T_new = n1;
  a.o = s0;
  a.src_t0 = t0;
  a.pos0 = p;
  pl->seg[0] = a;
  pl->nseg = 1;
  if (n1 < n) {                                      // wraps to row 0
    a.T_new = n - n1;
    a.o = 0;
    a.src_t0 = t0 + n1;
    a.pos0 = p + n1;
    pl->seg[1] = a;
    pl->nseg = 2;
  }
  pl->t0 = t0;
  return SA_OK;
}
// Bookkeeping after an append of T_new rows was enqueued.
static void appended(sa_kv_cache* c, int T_new) {
  c->stamp += 1;
  if (!c->ring && c->offset < c->high_water) c->rewrites.emplace_back(c->stamp, c->offset);
  c->offset += T_new;
  if (c->offset > c->high_water) c->high_water = c->offset;
}
}  // namespace

int kv_cache_append(sa_kv_cache* c, const void* k_rot, const void* v, int T_new, void* stream) {
  AppendPlan pl;
  int st = append_plan(c, k_rot, v, T_new, &pl);
  if (st != SA_OK) return st;
  for (int i = 0; i < pl.nseg; ++i) {
    hipError_t e = launch_append(pl.seg[i], elt_bytes(c->dtype), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "append launch");
  }
  appended(c, T_new);
  return ok();
}

int kv_cache_append_rope(sa_kv_cache* c, const void* k, const void* v, int T_new, const sa_yarn* y,
                         void* stream) {
  return kv_cache_append_rope_qk(c, nullptr, nullptr, 0, k, v, T_new, y, stream);
}

int kv_cache_append_rope_qk(sa_kv_cache* c, const void* q, void* q_rot, int n_q, const void* k,
                            const void* v, int T_new, const sa_yarn* y, void* stream) {
  AppendRopeArgs a;
  memset(&a, 0, sizeof a);
  AppendPlan pl;
  int st = append_plan(c, k, v, T_new, &pl);
  if (st != SA_OK) return st;
  if (q || q_rot) {
    if (!q || !q_rot) return fail(SA_ERR_ARG, "q and q_rot must both be given");
    if (misaligned(q) || misaligned(q_rot)) return fail(SA_ERR_ARG, "q and q_rot must be 16-byte aligned");
    if (n_q <= 0) return fail(SA_ERR_ARG, "n_q must be positive");
    const char* qb = static_cast<const char*>(q);
    const char* rb = static_cast<const char*>(q_rot);
    const int64_t bytes = (int64_t)c->B * T_new * n_q * c->d_h * elt_bytes(c->dtype);
    if (qb != rb && qb < rb + bytes && rb < qb + bytes)
      return fail(SA_ERR_ARG, "q and q_rot overlap without being the same buffer");
    a.q_src = q;
    a.q_dst = q_rot;
    a.n_q = n_q;
  }
  if (c->dtype == SA_BF16 && c->d_h % 16)
    return fail(SA_ERR_SHAPE, "bf16 rotate-and-append needs d_h %% 16 == 0, got %d", c->d_h);
  st = yarn_table(y, c->d_h, a.inv_freq, &a.conc);
  if (st != SA_OK) return st;
  const int eb = elt_bytes(c->dtype);
  if (a.q_src && pl.t0 > 0) {
    // a ring keeps only the last rows of this append, but every query row is
    // rotated: Q goes through yarn_rope's kernel (same bits) on its own
    RopeArgs r;
    memset(&r, 0, sizeof r);
    r.src = a.q_src;
    r.x = a.q_dst;
    r.offset = c->offset;
    r.BT = c->B * T_new;
    r.T = T_new;
    r.H = a.n_q;
    r.d = c->d_h;
    r.conc = a.conc;
    memcpy(r.inv_freq, a.inv_freq, sizeof r.inv_freq);
    if ((int64_t)c->B * T_new > INT32_MAX) return fail(SA_ERR_ARG, "B*T_new too large");
    hipError_t e = launch_rope(r, eb, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "rope launch");
    a.q_src = nullptr;
    a.q_dst = nullptr;
  }
  for (int i = 0; i < pl.nseg; ++i) {
    a.ap = pl.seg[i];
    hipError_t e = launch_append_rope(a, eb, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "append launch");
  }
  appended(c, T_new);
  return ok();
}

int kv_cache_snapshot(const sa_kv_cache* c, sa_kv_snapshot* out) {
  if (!c || !out) return fail(SA_ERR_ARG, "null argument");
  out->offset = c->offset;
  out->cache_id = c->id;
  out->stamp = c->stamp;
  return ok();
}

int kv_cache_restore(sa_kv_cache* c, const sa_kv_snapshot* snap) {
  if (!c || !snap) return fail(SA_ERR_ARG, "null argument");
  if (snap->cache_id != c->id) return fail(SA_ERR_SNAPSHOT, "snapshot belongs to another cache");
  if (snap->stamp > c->stamp || snap->offset < 0 || snap->offset > c->high_water)
    return fail(SA_ERR_SNAPSHOT, "snapshot is not from this cache's history");
  if (c->ring && snap->stamp != c->stamp)
    return fail(SA_ERR_SNAPSHOT, "a ring overwrites its rows as it goes: rows were appended since "
                                 "the snapshot (restore a ring with kv_ring_load)");
  for (const auto& w : c->rewrites)
    if (w.first > snap->stamp && w.second < snap->offset)
      return fail(SA_ERR_SNAPSHOT, "row %lld below the snapshot offset %lld was rewritten",
                  (long long)w.second, (long long)snap->offset);
  c->offset = snap->offset;
  return ok();
}

namespace {
static bool same_layout(const sa_kv_cache* a, const sa_kv_cache* b) {
  return a->B == b->B && a->n_kv == b->n_kv && a->d_h == b->d_h;
}
static CopyRowsArgs copy_args(const sa_kv_cache* src, sa_kv_cache* dst, int64_t p0, int n) {
  CopyRowsArgs a;
  a.ks = src->k;
  a.vs = src->v;
  a.kd = dst->k;
  a.vd = dst->v;
  a.Cs = src->capacity;
  a.Cd = dst->capacity;
  a.base_s = src->base;
  a.base_d = dst->base;
  a.ring_s = src->ring;
  a.ring_d = dst->ring;
  a.p0 = p0;
  a.n = n;
  a.B = src->B;
  a.n_kv = src->n_kv;
  a.d = src->d_h;
  return a;
}
}  // namespace

int kv_ring_stage(sa_kv_cache* stage, const sa_kv_cache* ring, void* stream) {
  if (!stage || !ring) return fail(SA_ERR_ARG, "null argument");
  if (!ring->ring || stage->ring)
    return fail(SA_ERR_ARG, "kv_ring_stage copies a ring cache into a linear one");
  if (!same_layout(stage, ring)) return fail(SA_ERR_SHAPE, "stage and ring differ in B/n_kv/d_h");
  if (stage->dtype != ring->dtype) return fail(SA_ERR_DTYPE, "stage and ring differ in dtype");
  const int64_t n_prev = std::min<int64_t>(ring->offset, ring->capacity - 1);
  if (n_prev > stage->capacity)
    return fail(SA_ERR_CAPACITY, "stage of %lld rows cannot hold the ring's %lld rows",
                (long long)stage->capacity, (long long)n_prev);
  if (n_prev > 0) {
    sa_kv_cache tmp = *stage;          // the destination mapping after staging
    tmp.base = ring->offset - n_prev;
    hipError_t e = launch_copy_rows(copy_args(ring, &tmp, ring->offset - n_prev, (int)n_prev),
                                    elt_bytes(ring->dtype), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "ring copy launch");
  }
  stage->base = ring->offset - n_prev;
  stage->offset = ring->offset;
  stage->high_water = ring->offset;
  stage->rewrites.clear();
  stage->id = g_next_id.fetch_add(1);   // a new history: older snapshots are refused
  stage->stamp = 0;
  stage->staged_from = ring->id;
  stage->staged_stamp = ring->stamp;
  return ok();
}

int kv_ring_commit(sa_kv_cache* ring, sa_kv_cache* stage, void* stream) {
  if (!stage || !ring) return fail(SA_ERR_ARG, "null argument");
  if (!ring->ring || stage->ring)
    return fail(SA_ERR_ARG, "kv_ring_commit copies a linear stage cache into a ring");
  if (stage->staged_from != ring->id || stage->staged_stamp != ring->stamp)
    return fail(SA_ERR_SNAPSHOT, "the stage was not staged from this ring, or the ring changed since");
  if (stage->offset < ring->offset)
    return fail(SA_ERR_SNAPSHOT, "the stage (offset %lld) is behind the ring (offset %lld)",
                (long long)stage->offset, (long long)ring->offset);
  const int64_t p0 = std::max(ring->offset, stage->offset - ring->capacity);
  const int n = (int)(stage->offset - p0);
  if (n > 0) {
    hipError_t e = launch_copy_rows(copy_args(stage, ring, p0, n), elt_bytes(ring->dtype),
                                    (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "ring copy launch");
  }
  ring->stamp += 1;
  ring->offset = stage->offset;
  if (ring->offset > ring->high_water) ring->high_water = ring->offset;
  stage->staged_stamp = ring->stamp;
  return ok();
}

namespace {
static int ring_copy(const sa_kv_cache* ring, void* kd, const void* ks, void* vd, const void* vs,
              void* stream) {
  const size_t bytes = (size_t)ring->B * ring->capacity * ring->n_kv * ring->d_h * elt_bytes(ring->dtype);
  hipError_t e = hipMemcpyAsync(kd, ks, bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream);
  if (e == hipSuccess) e = hipMemcpyAsync(vd, vs, bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "ring copy");
  return SA_OK;
}
}  // namespace

int kv_ring_save(const sa_kv_cache* ring, void* k_save, void* v_save, sa_kv_snapshot* out,
                 void* stream) {
  if (!ring || !k_save || !v_save || !out) return fail(SA_ERR_ARG, "null argument");
  if (!ring->ring) return fail(SA_ERR_ARG, "kv_ring_save takes a ring cache");
  if (misaligned(k_save) || misaligned(v_save))
    return fail(SA_ERR_ARG, "save buffers must be 16-byte aligned");
  int st = ring_copy(ring, k_save, ring->k, v_save, ring->v, stream);
  if (st != SA_OK) return st;
  out->offset = ring->offset;
  out->cache_id = ring->id;
  out->stamp = ring->stamp;
  return ok();
}

int kv_ring_load(sa_kv_cache* ring, const void* k_save, const void* v_save,
                 const sa_kv_snapshot* snap, void* stream) {
  if (!ring || !k_save || !v_save || !snap) return fail(SA_ERR_ARG, "null argument");
  if (!ring->ring) return fail(SA_ERR_ARG, "kv_ring_load takes a ring cache");
  if (snap->cache_id != ring->id) return fail(SA_ERR_SNAPSHOT, "snapshot belongs to another cache");
  if (snap->offset < 0 || snap->stamp > ring->stamp)
    return fail(SA_ERR_SNAPSHOT, "snapshot is not from this cache's history");
  if (misaligned(k_save) || misaligned(v_save))
    return fail(SA_ERR_ARG, "save buffers must be 16-byte aligned");
  int st = ring_copy(ring, ring->k, k_save, ring->v, v_save, stream);
  if (st != SA_OK) return st;
  ring->stamp += 1;
  ring->offset = snap->offset;
  return ok();
}

static int check_attn(const void* q, const sa_kv_cache* c, const float* sinks, const void* out,
                      int B, int T_q, int n_q, int n_kv, int d_h) {
  if (!q || !c || !sinks || !out) return fail(SA_ERR_ARG, "null argument");
  if (misaligned(q) || misaligned(out)) return fail(SA_ERR_ARG, "q and out must be 16-byte aligned");
  if (B <= 0 || T_q < 0 || n_q <= 0 || n_kv <= 0 || d_h <= 0)
    return fail(SA_ERR_ARG, "non-positive size");
  if (n_q % n_kv) return fail(SA_ERR_SHAPE, "n_q %d is not a multiple of n_kv %d", n_q, n_kv);
  if (B != c->B || n_kv != c->n_kv || d_h != c->d_h)
    return fail(SA_ERR_SHAPE, "B/n_kv/d_h (%d/%d/%d) differ from the cache's (%d/%d/%d)", B, n_kv,
                d_h, c->B, c->n_kv, c->d_h);
  return SA_OK;
}

namespace {
// Shared by the prefill entry points; yarn != nullptr: q is unrotated and the
// bf16 kernel rotates it first.
static int prefill_common(const void* q, const sa_kv_cache* c, const float* sinks, void* out, int B,
                   int T_q, int n_q, int n_kv, int d_h, int window, float sm_scale,
                   int64_t q_offset, const sa_yarn* yarn, void* stream) {
  int st = check_attn(q, c, sinks, out, B, T_q, n_q, n_kv, d_h);
  if (st != SA_OK) return st;
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(SA_ERR_ARG, "sm_scale must be finite and > 0");
  if (c->ring)
    return fail(SA_ERR_ARG, "a ring cache serves decode; attend a chunk through a stage cache "
                            "(kv_ring_stage)");
  if (q_offset < 0 || q_offset + T_q > c->offset)
    return fail(SA_ERR_CAPACITY, "queries [%lld, %lld) reach past the %lld rows in the cache",
                (long long)q_offset, (long long)(q_offset + T_q), (long long)c->offset);
  {
    const int64_t lowest = window > 0 ? std::max<int64_t>(0, q_offset - window + 1) : 0;
    if (lowest < c->base)
      return fail(SA_ERR_CAPACITY, "keys from position %lld are needed but the cache starts at %lld",
                  (long long)lowest, (long long)c->base);
  }
  const int q_mult = n_q / n_kv;
  if (c->dtype == SA_BF16) {
    if (d_h != 64 && d_h != 96 && d_h != 128)
      return fail(SA_ERR_SHAPE, "bf16 attention supports d_h in {64, 96, 128}, got %d", d_h);
    if (q_mult > 128) return fail(SA_ERR_SHAPE, "n_q/n_kv must be <= 128");
    if (c->capacity > INT32_MAX)   // the kernel keeps key positions in 32 bits
      return fail(SA_ERR_SHAPE, "bf16 prefill needs a capacity below 2^31 rows");
  }
  RopeTab rt;
  rt.pos_base = c->base;
  if (yarn) {
    if (c->dtype != SA_BF16) return fail(SA_ERR_DTYPE, "in-kernel Q rotation needs a bf16 cache");
    st = yarn_table(yarn, d_h, rt.inv_freq, &rt.conc);
    if (st != SA_OK) return st;
  }
  if ((int64_t)B * T_q * n_q > INT32_MAX) return fail(SA_ERR_ARG, "B*T_q*n_q too large");
  if (T_q == 0) return ok();
  AttnArgs a;
  a.q = q;
  a.kc = c->k;
  a.vc = c->v;
  a.sinks = sinks;
  a.out = out;
  a.B = B;
  a.T_q = T_q;
  a.n_q = n_q;
  a.n_kv = n_kv;
  a.d = d_h;
  a.q_mult = q_mult;
  a.window = window > 0 ? window : 0;
  a.C = c->capacity;
  a.q_offset = q_offset - c->base;
  a.sm_scale = sm_scale;
  hipError_t e = c->dtype == SA_BF16
                     ? launch_prefill_bf16(a, yarn ? &rt : nullptr, (hipStream_t)stream)
                     : launch_attn_rows_f32(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return ok();
}
}  // namespace

int sinkattn_prefill(const void* q, const sa_kv_cache* c, const float* sinks, void* out, int B,
                     int T_q, int n_q, int n_kv, int d_h, int window, float sm_scale,
                     int64_t q_offset, void* stream) {
  return prefill_common(q, c, sinks, out, B, T_q, n_q, n_kv, d_h, window, sm_scale, q_offset,
                        nullptr, stream);
}

int sinkattn_prefill_rope(const void* q, const sa_kv_cache* c, const float* sinks, void* out,
                          int B, int T_q, int n_q, int n_kv, int d_h, int window, float sm_scale,
                          int64_t q_offset, const sa_yarn* y, void* stream) {
  if (!y) return fail(SA_ERR_ARG, "yarn parameters are null");
  return prefill_common(q, c, sinks, out, B, T_q, n_q, n_kv, d_h, window, sm_scale, q_offset, y,
                        stream);
}

size_t sinkattn_qkv_workspace_bytes(int T, int d_h) {
  if (T <= 0 || d_h <= 0 || d_h % 2) return 0;
  return (size_t)T * (size_t)(d_h / 2) * 16;
}

int sinkattn_qkv_rope_append(sa_kv_cache* c, const void* x, const void* w_qkv, const void* b_qkv,
                             void* q_rot, int B, int T, int d_model, int n_q, const sa_yarn* y,
                             void* workspace, size_t ws_bytes, void* stream) {
  if (!c || !x || !w_qkv || !b_qkv || !q_rot || !workspace) return fail(SA_ERR_ARG, "null argument");
  if (misaligned(x) || misaligned(w_qkv) || misaligned(b_qkv) || misaligned(q_rot) ||
      misaligned(workspace))
    return fail(SA_ERR_ARG, "x, w_qkv, b_qkv, q_rot and workspace must be 16-byte aligned");
  if (c->ring)
    return fail(SA_ERR_ARG, "the fused projection appends to a linear cache (a stage for a ring)");
  if (c->dtype != SA_BF16) return fail(SA_ERR_DTYPE, "the fused projection is bf16 only");
  if (B <= 0 || T <= 0 || n_q <= 0 || d_model <= 0) return fail(SA_ERR_ARG, "non-positive size");
  if (B != c->B) return fail(SA_ERR_SHAPE, "B %d differs from the cache's %d", B, c->B);
  const int d = c->d_h;
  if (d != 64 && d != 96 && d != 128)
    return fail(SA_ERR_SHAPE, "the fused projection supports d_h in {64, 96, 128}, got %d", d);
  if (d_model % 64) return fail(SA_ERR_SHAPE, "d_model must be a multiple of 64, got %d", d_model);
  const int64_t M = (int64_t)B * T;
  const int64_t dqkv = (int64_t)d * (n_q + 2 * c->n_kv);
  if (M * d_model > UINT32_MAX || dqkv * d_model > UINT32_MAX || M * n_q > INT32_MAX)
    return fail(SA_ERR_ARG, "B*T*d_model or d_qkv*d_model too large");
  const int64_t row = c->offset - c->base;
  if (row + T > c->capacity)
    return fail(SA_ERR_CAPACITY, "append of %d rows at row %lld exceeds capacity %lld", T,
                (long long)row, (long long)c->capacity);
  const size_t need = sinkattn_qkv_workspace_bytes(T, d);
  if (ws_bytes < need) return fail(SA_ERR_ARG, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  QkvArgs a;
  memset(&a, 0, sizeof a);
  int st = yarn_table(y, d, a.inv_freq, &a.conc);
  if (st != SA_OK) return st;
  a.x = x;
  a.w = w_qkv;
  a.bias = b_qkv;
  a.q_rot = q_rot;
  a.kc = c->k;
  a.vc = c->v;
  a.tab = reinterpret_cast<double2*>(workspace);
  a.B = B;
  a.T = T;
  a.d_model = d_model;
  a.n_q = n_q;
  a.n_kv = c->n_kv;
  a.d = d;
  a.C = c->capacity;
  a.row0 = row;
  a.pos0 = c->offset;
  hipError_t e = launch_qkv_rope_append(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fused projection launch");
  appended(c, T);
  return ok();
}

// ---- MoE layer
namespace {
static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
struct MoeLayout {          // byte offsets of the workspace sections
  size_t logits, ids, weights, counts, offsets, expert_start, tile_start, rows, h, hs, out, total;
};
static MoeLayout moe_layout(int N, int d_model, int E, int k, int ffn, int ffn_s) {
  MoeLayout L;
  const size_t nblk = ((size_t)N + 255) / 256;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align256(bytes); return at; };
  L.logits = take((size_t)N * E * 2);
  L.ids = take((size_t)N * k * 4);
  L.weights = take((size_t)N * k * 4);
  L.counts = take(nblk * E * 4);
  L.offsets = take(nblk * E * 4);
  L.expert_start = take((size_t)(E + 1) * 4);
  L.tile_start = take((size_t)(E + 1) * 4);
  L.rows = take((size_t)N * k * 4);
  L.h = take((size_t)N * k * ffn * 2);
  L.hs = take((size_t)N * ffn_s * 2);
  L.out = take((size_t)N * (k + 1) * d_model * 4);
  L.total = o;
  return L;
}
static int moe_check(int N, int d_model, int E, int k) {
  if (N <= 0 || d_model <= 0) return fail(SA_ERR_ARG, "non-positive size");
  if (E < 1 || E > 64) return fail(SA_ERR_SHAPE, "E must be in [1, 64], got %d", E);
  if (k < 1 || k > 8 || k > E) return fail(SA_ERR_SHAPE, "k must be in [1, min(8, E)], got %d", k);
  if (d_model % 64) return fail(SA_ERR_SHAPE, "d_model must be a multiple of 64, got %d", d_model);
  if ((int64_t)N * d_model > UINT32_MAX || (int64_t)N * k > INT32_MAX)
    return fail(SA_ERR_ARG, "N too large");
  if (((int64_t)N + 255) / 256 * E * 4 > 65536)     // per-block counts staged in LDS
    return fail(SA_ERR_ARG, "N * E too large for the dispatch scan (N/256 * E <= 16384)");
  return SA_OK;
}
}  // namespace

size_t moe_workspace_bytes(int N, int d_model, int E, int k, int ffn, int ffn_shared) {
  if (N <= 0 || d_model <= 0 || E <= 0 || k <= 0 || ffn < 0 || ffn_shared < 0) return 0;
  return moe_layout(N, d_model, E, k, ffn, ffn_shared).total;
}

int moe_route(const void* x, int N, int d_model, const void* w_router, int E, int k, void* logits,
              int32_t* expert_ids, float* weights, void* stream) {
  if (!x || !w_router || !logits || !expert_ids || !weights) return fail(SA_ERR_ARG, "null argument");
  if (misaligned(x) || misaligned(w_router)) return fail(SA_ERR_ARG, "x and w_router must be 16-byte aligned");
  int st = moe_check(N, d_model, E, k);
  if (st != SA_OK) return st;
  MoeArgs a;
  memset(&a, 0, sizeof a);
  a.x = x;
  a.w_router = w_router;
  a.N = N;
  a.d_model = d_model;
  a.E = E;
  a.k = k;
  a.logits = logits;
  a.ids = expert_ids;
  a.weights = weights;
  hipError_t e = launch_moe_route(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "router launch");
  return ok();
}

size_t moe_dispatch_workspace_bytes(int N, int E) {
  if (N <= 0 || E <= 0) return 0;
  const size_t nblk = ((size_t)N + 255) / 256;
  return 2 * align256(nblk * E * 4) + align256((size_t)(E + 1) * 4);
}

int moe_dispatch(const int32_t* expert_ids, int N, int E, int k, int32_t* rows,
                 int32_t* expert_start, void* workspace, size_t ws_bytes, void* stream) {
  if (!expert_ids || !rows || !expert_start || !workspace) return fail(SA_ERR_ARG, "null argument");
  if (misaligned(workspace)) return fail(SA_ERR_ARG, "workspace must be 16-byte aligned");
  if (N <= 0) return fail(SA_ERR_ARG, "non-positive size");
  if (E < 1 || E > 64 || k < 1 || k > 8 || k > E) return fail(SA_ERR_SHAPE, "need 1 <= k <= min(8, E), E <= 64");
  if ((int64_t)N * k > INT32_MAX) return fail(SA_ERR_ARG, "N too large");
  if (((int64_t)N + 255) / 256 * E * 4 > 65536)
    return fail(SA_ERR_ARG, "N * E too large for the dispatch scan (N/256 * E <= 16384)");
  const size_t need = moe_dispatch_workspace_bytes(N, E);
  if (ws_bytes < need) return fail(SA_ERR_ARG, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  const size_t nblk = ((size_t)N + 255) / 256;
  char* w = static_cast<char*>(workspace);
  MoeArgs a;
  memset(&a, 0, sizeof a);
  a.N = N;
  a.E = E;
  a.k = k;
  a.ids = const_cast<int32_t*>(expert_ids);
  a.counts = reinterpret_cast<int32_t*>(w);
  a.offsets = reinterpret_cast<int32_t*>(w + align256(nblk * E * 4));
  a.tile_start = reinterpret_cast<int32_t*>(w + 2 * align256(nblk * E * 4));
  a.expert_start = expert_start;
  a.rows = rows;
  hipError_t e = launch_moe_dispatch(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "dispatch launch");
  return ok();
}

int moe_layer(const void* x, int N, int d_model, const void* w_router, int E, int k,
              const void* w13, const void* w2, int ffn, const void* w13_shared,
              const void* w2_shared, int ffn_shared, void* y, void* workspace, size_t ws_bytes,
              void* stream) {
  if (!x || !w_router || !w13 || !w2 || !y || !workspace) return fail(SA_ERR_ARG, "null argument");
  if (misaligned(x) || misaligned(w_router) || misaligned(w13) || misaligned(w2) || misaligned(y) ||
      misaligned(workspace))
    return fail(SA_ERR_ARG, "pointers must be 16-byte aligned");
  int st = moe_check(N, d_model, E, k);
  if (st != SA_OK) return st;
  if (ffn <= 0 || ffn % 128) return fail(SA_ERR_SHAPE, "ffn must be a positive multiple of 128, got %d", ffn);
  const bool shared = ffn_shared > 0;
  if (shared) {
    if (!w13_shared || !w2_shared) return fail(SA_ERR_ARG, "shared expert weights are null");
    if (misaligned(w13_shared) || misaligned(w2_shared)) return fail(SA_ERR_ARG, "pointers must be 16-byte aligned");
    if (ffn_shared % 128) return fail(SA_ERR_SHAPE, "ffn_shared must be a multiple of 128, got %d", ffn_shared);
  } else if (ffn_shared < 0 || w13_shared || w2_shared) {
    return fail(SA_ERR_ARG, "no shared expert: ffn_shared = 0 and null shared weights");
  }
  if ((int64_t)N * k * ffn > UINT32_MAX || (int64_t)N * ffn_shared > UINT32_MAX ||
      (int64_t)2 * ffn * d_model > UINT32_MAX || (int64_t)2 * ffn_shared * d_model > UINT32_MAX)
    return fail(SA_ERR_ARG, "sizes too large");
  const MoeLayout L = moe_layout(N, d_model, E, k, ffn, shared ? ffn_shared : 0);
  if (ws_bytes < L.total) return fail(SA_ERR_ARG, "workspace of %zu bytes needed, %zu given", L.total, ws_bytes);
  char* w = static_cast<char*>(workspace);
  MoeArgs a;
  memset(&a, 0, sizeof a);
  a.x = x;
  a.w_router = w_router;
  a.N = N;
  a.d_model = d_model;
  a.E = E;
  a.k = k;
  a.logits = w + L.logits;
  a.ids = reinterpret_cast<int32_t*>(w + L.ids);
  a.weights = reinterpret_cast<float*>(w + L.weights);
  a.counts = reinterpret_cast<int32_t*>(w + L.counts);
  a.offsets = reinterpret_cast<int32_t*>(w + L.offsets);
  a.expert_start = reinterpret_cast<int32_t*>(w + L.expert_start);
  a.tile_start = reinterpret_cast<int32_t*>(w + L.tile_start);
  a.rows = reinterpret_cast<int32_t*>(w + L.rows);
  a.out_slots = reinterpret_cast<float*>(w + L.out);
  a.y = y;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_moe_route(a, s);
  if (e == hipSuccess) e = launch_moe_dispatch(a, s);
  if (e == hipSuccess) {
    MoeGroup g{w13, w2, w + L.h, ffn, 0};
    e = launch_moe_experts(a, g, false, s);
  }
  if (e == hipSuccess && shared) {      // the shared expert's down pass also combines
    MoeGroup g{w13_shared, w2_shared, w + L.hs, ffn_shared, 1};
    e = launch_moe_experts(a, g, true, s);
  }
  if (e == hipSuccess && !shared) e = launch_moe_combine(a, k, s);
  if (e != hipSuccess) return hip_fail(e, "moe launch");
  return ok();
}

namespace {
struct SampleLayout {
  size_t zp, cmax, carg, hcount, hmass, cand, ncand, rmass, kmass, total;
};
SampleLayout sample_layout(int B, int V) {
  const size_t C = ((size_t)V + kSampleChunk - 1) / kSampleChunk;
  SampleLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align256(bytes); return at; };
  L.zp = take((size_t)B * (((size_t)V + 63) / 64 * 64) * 4);
  L.cmax = take((size_t)B * C * 4);
  L.carg = take((size_t)B * C * 4);
  L.hcount = take((size_t)B * kSampleHist * 4);
  L.hmass = take((size_t)B * kSampleHist * 8);
  L.cand = take((size_t)B * kSampleCap * 8);
  L.ncand = take((size_t)B * 4);
  L.rmass = take((size_t)B * C * 8);
  L.kmass = take((size_t)B * C * 8);
  L.total = o;
  return L;
}
int sample_shape(int B, int V) {
  if (B < 1 || B > 65535) return fail(SA_ERR_SHAPE, "B must be in [1, 65535], got %d", B);
  if (V < 1 || V > kSampleMaxV) return fail(SA_ERR_SHAPE, "V must be in [1, %d], got %d", kSampleMaxV, V);
  return SA_OK;
}
}  // namespace

int sample_count_tokens(const int32_t* ids, int B, int H, int64_t ids_stride, int32_t* counts, int V,
                        void* stream) {
  if (!counts || (H > 0 && !ids)) return fail(SA_ERR_ARG, "null argument");
  int st = sample_shape(B, V);
  if (st != SA_OK) return st;
  if (H < 0 || ids_stride < H) return fail(SA_ERR_ARG, "need H >= 0 and ids_stride >= H");
  if (H == 0) return ok();
  hipError_t e = launch_sample_count(ids, B, H, ids_stride, counts, V, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "count launch");
  return ok();
}

size_t sample_workspace_bytes(int B, int V) {
  if (B < 1 || B > 65535 || V < 1 || V > kSampleMaxV) return 0;
  return sample_layout(B, V).total;
}

int sample_tokens(const float* logits, int B, int V, int64_t logits_stride, const float* bias,
                  int64_t bias_stride, int32_t* counts, const sa_sample_params* params, const float* u,
                  int update_counts, int32_t* tokens, int32_t* n_kept, float* processed, void* workspace,
                  size_t ws_bytes, void* stream) {
  if (!logits || !params || !u || !tokens || !workspace) return fail(SA_ERR_ARG, "null argument");
  int st = sample_shape(B, V);
  if (st != SA_OK) return st;
  if (logits_stride < V) return fail(SA_ERR_ARG, "logits_stride must be >= V");
  if (bias && bias_stride != 0 && bias_stride < V) return fail(SA_ERR_ARG, "bias_stride must be 0 or >= V");
  if (update_counts && !counts) return fail(SA_ERR_ARG, "update_counts needs counts");
  if (misaligned(workspace)) return fail(SA_ERR_ARG, "workspace must be 16-byte aligned");
  const SampleLayout L = sample_layout(B, V);
  if (ws_bytes < L.total) return fail(SA_ERR_ARG, "workspace of %zu bytes needed, %zu given", L.total, ws_bytes);
  char* w = static_cast<char*>(workspace);
  SampleArgs a;
  memset(&a, 0, sizeof a);
  a.logits = logits;
  a.logits_stride = logits_stride;
  a.bias = bias;
  a.bias_stride = bias ? bias_stride : 0;
  a.counts = counts;
  a.params = params;
  a.u = u;
  a.tokens = tokens;
  a.n_kept = n_kept;
  a.processed = processed;
  a.zp = reinterpret_cast<float*>(w + L.zp);
  a.zs = ((int64_t)V + 63) / 64 * 64;
  a.chunk_max = reinterpret_cast<float*>(w + L.cmax);
  a.chunk_arg = reinterpret_cast<int32_t*>(w + L.carg);
  a.hist_count = reinterpret_cast<uint32_t*>(w + L.hcount);
  a.hist_mass = reinterpret_cast<unsigned long long*>(w + L.hmass);
  a.cand = reinterpret_cast<unsigned long long*>(w + L.cand);
  a.ncand = reinterpret_cast<uint32_t*>(w + L.ncand);
  a.chunk_mass = reinterpret_cast<unsigned long long*>(w + L.rmass);
  a.chunk_kmass = reinterpret_cast<unsigned long long*>(w + L.kmass);
  a.B = B;
  a.V = V;
  a.C = (V + kSampleChunk - 1) / kSampleChunk;
  a.update_counts = update_counts ? 1 : 0;
  hipError_t e = launch_sample(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sample launch");
  return ok();
}

size_t sinkattn_decode_workspace_bytes(int B, int n_q, int n_kv, int d_h, int64_t capacity) {
  if (B <= 0 || n_q <= 0 || n_kv <= 0 || d_h <= 0 || capacity <= 0 || n_q % n_kv) return 0;
  const int64_t S = decode_max_splits(B, n_kv, capacity);
  return (size_t)((int64_t)B * n_q * S * (d_h + 2) * 4);
}

}  // extern "C"

namespace {
// The decode launch behind both decode entry points.  With a caller
// workspace (ws_static false) it must hold the bound for the cache's whole
// capacity; with ws_static the partials go to this library's static device
// array (below), which must hold what this call's split count needs.
// step != nullptr: a fused step -- q holds the unrotated Q, and the token's
// row (not yet in the cache: c->offset is the token's position) is written
// by the kernels; the caller fills step's rotation fields and does the
// bookkeeping after a successful launch.
int decode_impl(const void* q, const sa_kv_cache* c, const float* sinks, void* out, int B,
                int n_q, int n_kv, int d_h, int window, float sm_scale, void* workspace,
                size_t ws_bytes, bool ws_static, StepArgs* step, void* stream) {
  int st = check_attn(q, c, sinks, out, B, 1, n_q, n_kv, d_h);
  if (st != SA_OK) return st;
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(SA_ERR_ARG, "sm_scale must be finite and > 0");
  const int64_t offset = c->offset + (step ? 1 : 0);     // rows once the token's is in
  if (offset < 1) return fail(SA_ERR_CAPACITY, "decode needs the step's row appended first");
  // rows handed to the kernel: a ring holds exactly the band (every live
  // slot is allowed, so it is attended as min(offset, W) unmasked rows); a
  // linear cache holds position p at row p - base
  int64_t q_row, win;
  if (c->ring) {
    if (window != c->capacity)
      return fail(SA_ERR_ARG, "a ring of %lld rows serves a band of exactly that width (window %d)",
                  (long long)c->capacity, window);
    q_row = std::min(offset, c->capacity) - 1;
    win = 0;
  } else {
    const int64_t lowest = window > 0 ? std::max<int64_t>(0, offset - window) : 0;
    if (lowest < c->base)
      return fail(SA_ERR_CAPACITY, "keys from position %lld are needed but the cache starts at %lld",
                  (long long)lowest, (long long)c->base);
    q_row = offset - 1 - c->base;
    win = window > 0 ? window : 0;
  }
  if (step) {
    if (c->dtype != SA_BF16) return fail(SA_ERR_DTYPE, "the fused decode step needs a bf16 cache");
    step->row = c->ring ? c->offset % c->capacity : c->offset - c->base;
    step->pos = c->offset;
  }
  const int q_mult = n_q / n_kv;
  AttnArgs a;
  a.q = q;
  a.kc = c->k;
  a.vc = c->v;
  a.sinks = sinks;
  a.out = out;
  a.B = B;
  a.T_q = 1;
  a.n_q = n_q;
  a.n_kv = n_kv;
  a.d = d_h;
  a.q_mult = q_mult;
  a.window = (int)win;
  a.C = c->capacity;
  a.q_offset = q_row;
  a.sm_scale = sm_scale;
  hipError_t e;
  if (c->dtype == SA_BF16) {
    if (d_h != 64 && d_h != 96 && d_h != 128)
      return fail(SA_ERR_SHAPE, "bf16 attention supports d_h in {64, 96, 128}, got %d", d_h);
    if (q_mult > 16) return fail(SA_ERR_SHAPE, "bf16 decode needs n_q/n_kv <= 16");
    if (c->capacity > INT32_MAX)   // the kernels keep 32-key block indices in 32 bits
      return fail(SA_ERR_SHAPE, "bf16 decode needs a capacity below 2^31 rows");
    const int64_t rows = q_row + 1;
    const int64_t span = a.window > 0 ? std::min<int64_t>(a.window, rows) : rows;
    DecodeArgs da;
    da.at = a;
    da.n_splits = decode_splits(B, n_kv, span);
    if (ws_static) {
      const size_t need =
          da.n_splits > 1 ? (size_t)((int64_t)B * n_q * da.n_splits * (d_h + 2) * 4) : 0;
      st = static_scratch(need, &workspace);
      if (st != SA_OK) return st;
    } else {
      const size_t need = sinkattn_decode_workspace_bytes(B, n_q, n_kv, d_h, c->capacity);
      if (!workspace || ws_bytes < need || misaligned(workspace))
        return fail(SA_ERR_ARG, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
    }
    da.ws = reinterpret_cast<float*>(workspace);
    e = step ? launch_decode_step_bf16(da, *step, (hipStream_t)stream)
             : launch_decode_bf16(da, (hipStream_t)stream);
  } else {
    e = launch_attn_rows_f32(a, (hipStream_t)stream);
  }
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}
}  // namespace

extern "C" {

int sinkattn_decode(const void* q, const sa_kv_cache* c, const float* sinks, void* out, int B,
                    int n_q, int n_kv, int d_h, int window, float sm_scale, void* workspace,
                    size_t ws_bytes, void* stream) {
  return decode_impl(q, c, sinks, out, B, n_q, n_kv, d_h, window, sm_scale, workspace, ws_bytes,
                     false, nullptr, stream);
}

int sinkattn_decode_step(sa_kv_cache* c, const void* q, void* q_rot, const void* k, const void* v,
                         const float* sinks, void* out, int B, int n_q, int n_kv, int d_h,
                         int window, float sm_scale, const sa_yarn* y, void* workspace,
                         size_t ws_bytes, void* stream) {
  // every check before anything is enqueued or recorded
  AppendPlan pl;
  int st = append_plan(c, k, v, 1, &pl);
  if (st != SA_OK) return st;
  if (!q || !out) return fail(SA_ERR_ARG, "null argument");
  const int64_t qbytes = (int64_t)B * n_q * d_h * 2;
  if (q_rot) {
    if (misaligned(q_rot)) return fail(SA_ERR_ARG, "q_rot must be 16-byte aligned");
    const char* r = static_cast<const char*>(q_rot);
    const char* a = static_cast<const char*>(q);
    const char* o = static_cast<const char*>(out);
    if (qbytes > 0 && ((r < a + qbytes && a < r + qbytes) || (r < o + qbytes && o < r + qbytes)))
      return fail(SA_ERR_ARG, "q_rot overlaps q or out");
  }
  StepArgs sp;
  memset(&sp, 0, sizeof sp);
  st = yarn_table(y, d_h, sp.inv_freq, &sp.conc);
  if (st != SA_OK) return st;
  sp.q_raw = q;
  sp.q_rot = q_rot;
  sp.k_raw = k;
  sp.v_raw = v;
  st = decode_impl(q, c, sinks, out, B, n_q, n_kv, d_h, window, sm_scale, workspace, ws_bytes,
                   false, &sp, stream);
  if (st != SA_OK) return st;
  appended(c, 1);
  return ok();
}

int sinkattn_decode_noalloc(const void* q, const sa_kv_cache* c, const float* sinks, void* out,
                            int B, int n_q, int n_kv, int d_h, int window, float sm_scale,
                            void* stream) {
  return decode_impl(q, c, sinks, out, B, n_q, n_kv, d_h, window, sm_scale, nullptr, 0, true,
                     nullptr, stream);
}

size_t sinkattn_decode_scratch_bytes(void) { return (size_t)SA_DECODE_SCRATCH_BYTES; }

}  // extern "C"
