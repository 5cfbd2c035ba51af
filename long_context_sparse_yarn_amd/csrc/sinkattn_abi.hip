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
#include <atomic>

#include "../../include/sinkattn.h"
#include "sa_kernels.h"

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

struct sa_kv_cache {
  void* k;
  void* v;
  int dtype;
  int B, n_kv, d_h;
  int64_t capacity;
  int64_t offset;
  uint64_t id;
  uint64_t stamp;
  // (stamp, first row) of appends that began below the high-water mark,
  // i.e. that may have overwritten rows some snapshot relies on.
  std::vector<std::pair<uint64_t, int64_t>> rewrites;
  int64_t high_water;
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

int kv_cache_create(sa_kv_cache** out, void* k, void* v, int dtype, int B, int64_t capacity,
                    int n_kv, int d_h, int64_t offset) {
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
  c->high_water = offset;
  c->id = g_next_id.fetch_add(1);
  c->stamp = 0;
  *out = c;
  return ok();
}

int kv_cache_destroy(sa_kv_cache* c) {
  if (!c) return fail(SA_ERR_ARG, "null cache");
  delete c;
  return ok();
}

int64_t kv_cache_offset(const sa_kv_cache* c) { return c ? c->offset : -1; }

namespace {
// Checks shared by the append entry points; fills the launch arguments.
int append_args(sa_kv_cache* c, const void* k, const void* v, int T_new, AppendArgs* a) {
  if (!c || !k || !v) return fail(SA_ERR_ARG, "null argument");
  if (misaligned(k) || misaligned(v)) return fail(SA_ERR_ARG, "k and v must be 16-byte aligned");
  if (T_new <= 0) return fail(SA_ERR_ARG, "T_new must be positive");
  if (c->offset + T_new > c->capacity)
    return fail(SA_ERR_CAPACITY, "append of %d rows at offset %lld exceeds capacity %lld", T_new,
                (long long)c->offset, (long long)c->capacity);
  a->k_src = k;
  a->v_src = v;
  a->kc = c->k;
  a->vc = c->v;
  a->B = c->B;
  a->T_new = T_new;
  a->n_kv = c->n_kv;
  a->d = c->d_h;
  a->C = c->capacity;
  a->o = c->offset;
  return SA_OK;
}
// Bookkeeping after an append of T_new rows was enqueued.
void appended(sa_kv_cache* c, int T_new) {
  c->stamp += 1;
  if (c->offset < c->high_water) c->rewrites.emplace_back(c->stamp, c->offset);
  c->offset += T_new;
  if (c->offset > c->high_water) c->high_water = c->offset;
}
}  // namespace

int kv_cache_append(sa_kv_cache* c, const void* k_rot, const void* v, int T_new, void* stream) {
  AppendArgs a;
  int st = append_args(c, k_rot, v, T_new, &a);
  if (st != SA_OK) return st;
  hipError_t e = launch_append(a, elt_bytes(c->dtype), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "append launch");
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
  int st = append_args(c, k, v, T_new, &a.ap);
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
  hipError_t e = launch_append_rope(a, elt_bytes(c->dtype), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "append launch");
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
  for (const auto& w : c->rewrites)
    if (w.first > snap->stamp && w.second < snap->offset)
      return fail(SA_ERR_SNAPSHOT, "row %lld below the snapshot offset %lld was rewritten",
                  (long long)w.second, (long long)snap->offset);
  c->offset = snap->offset;
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
int prefill_common(const void* q, const sa_kv_cache* c, const float* sinks, void* out, int B,
                   int T_q, int n_q, int n_kv, int d_h, int window, float sm_scale,
                   int64_t q_offset, const sa_yarn* yarn, void* stream) {
  int st = check_attn(q, c, sinks, out, B, T_q, n_q, n_kv, d_h);
  if (st != SA_OK) return st;
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(SA_ERR_ARG, "sm_scale must be finite and > 0");
  if (q_offset < 0 || q_offset + T_q > c->offset)
    return fail(SA_ERR_CAPACITY, "queries [%lld, %lld) reach past the %lld rows in the cache",
                (long long)q_offset, (long long)(q_offset + T_q), (long long)c->offset);
  const int q_mult = n_q / n_kv;
  if (c->dtype == SA_BF16) {
    if (d_h != 64 && d_h != 96 && d_h != 128)
      return fail(SA_ERR_SHAPE, "bf16 attention supports d_h in {64, 96, 128}, got %d", d_h);
    if (q_mult > 128) return fail(SA_ERR_SHAPE, "n_q/n_kv must be <= 128");
    if (c->capacity > INT32_MAX)   // the kernel keeps key positions in 32 bits
      return fail(SA_ERR_SHAPE, "bf16 prefill needs a capacity below 2^31 rows");
  }
  RopeTab rt;
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
  a.q_offset = q_offset;
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

size_t sinkattn_decode_workspace_bytes(int B, int n_q, int n_kv, int d_h, int64_t capacity) {
  if (B <= 0 || n_q <= 0 || n_kv <= 0 || d_h <= 0 || capacity <= 0 || n_q % n_kv) return 0;
  const int64_t S = decode_max_splits(B, n_kv, capacity);
  return (size_t)((int64_t)B * n_q * S * (d_h + 2) * 4);
}

int sinkattn_decode(const void* q, const sa_kv_cache* c, const float* sinks, void* out, int B,
                    int n_q, int n_kv, int d_h, int window, float sm_scale, void* workspace,
                    size_t ws_bytes, void* stream) {
  int st = check_attn(q, c, sinks, out, B, 1, n_q, n_kv, d_h);
  if (st != SA_OK) return st;
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(SA_ERR_ARG, "sm_scale must be finite and > 0");
  if (c->offset < 1) return fail(SA_ERR_CAPACITY, "decode needs the step's row appended first");
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
  a.window = window > 0 ? window : 0;
  a.C = c->capacity;
  a.q_offset = c->offset - 1;
  a.sm_scale = sm_scale;
  hipError_t e;
  if (c->dtype == SA_BF16) {
    if (d_h != 64 && d_h != 96 && d_h != 128)
      return fail(SA_ERR_SHAPE, "bf16 attention supports d_h in {64, 96, 128}, got %d", d_h);
    if (q_mult > 16) return fail(SA_ERR_SHAPE, "bf16 decode needs n_q/n_kv <= 16");
    const size_t need = sinkattn_decode_workspace_bytes(B, n_q, n_kv, d_h, c->capacity);
    if (!workspace || ws_bytes < need || misaligned(workspace))
      return fail(SA_ERR_ARG, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
    const int64_t span = a.window > 0 ? (a.window < c->offset ? a.window : c->offset) : c->offset;
    DecodeArgs da;
    da.at = a;
    da.ws = reinterpret_cast<float*>(workspace);
    da.n_splits = decode_splits(B, n_kv, span);
    e = launch_decode_bf16(da, (hipStream_t)stream);
  } else {
    e = launch_attn_rows_f32(a, (hipStream_t)stream);
  }
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

}  // extern "C"
