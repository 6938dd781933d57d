// Loop driver and C ABI (include/loop.h).
//
// The driver owns no device memory.  It turns the execution config into a
// schedule table, one entry per layer execution (stored layer, pass, kind,
// per-(layer, pass) cache slot), and walks it, enqueueing the kernels of every
// sublayer on the caller's stream.  Each shared layer's weights are read once
// per pass: the block [loop_start, loop_end) is walked n_passes times with the
// same weight pointers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/loop.h"
#include "abi_util.h"
#include "kernels.h"

namespace {
thread_local std::string g_err;

// Workspace of loop_decode_step_noalloc, for callers that cannot allocate.
// Every GPU the library runs on holds its own copy of this array until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in symbol): it uses the device address that
// hipGetSymbolAddress returned for the current device, kept per device below.
constexpr size_t NOALLOC_WS_BYTES = (size_t)64 << 20;
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[NOALLOC_WS_BYTES];

int lp_fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

namespace {

bool misaligned(const void* p) { return lp_misaligned(p); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Exec {
  int layer, pass, full, slot;
};

constexpr int LIN_CHUNK = 64;

}  // namespace

struct loop_model {
  loop_config cfg;
  std::vector<loop_layer_weights> layers;
  const void* embed;
  const float* final_norm;
  const void* head;
  std::vector<Exec> sched;
  int n_full = 0, n_lin = 0;
  int es = 4;
  int cu = 0;
  bool in_loop(int i) const { return i >= cfg.loop_start && i < cfg.loop_end; }
  int qkv_rows() const { return (cfg.n_heads + 2 * cfg.n_kv_heads) * cfg.head_dim; }
};

struct loop_state {
  const loop_model* m;
  char* base;
  size_t bytes;
  int batch, max_seq, S_max;
  std::vector<int> seq_len;     // positions each sequence holds (sequences may differ: ragged batch)
  // paged KV: each full-attention slot is a pool of n_pages pages of 64
  // positions; table [batch][table_stride] (caller-owned device memory) maps a
  // sequence's 64-position block to its page in every slot's pool
  int n_pages = 0;
  const int32_t* table = nullptr;
  int table_stride = 0;
  // the page table of the sequences from seq0 on (empty for a contiguous state)
  lk::KvPages pages(int seq0) const {
    return table ? lk::KvPages{table + (size_t)seq0 * table_stride, table_stride, n_pages} : lk::KvPages{};
  }
  // byte offset of sequence seq0's part of a K or V^T slot (0 for a paged pool, which all share)
  size_t kv_seq_off(int seq0, size_t per_seq) const { return table ? 0 : (size_t)seq0 * per_seq; }
  size_t pos_off = 0;           // int32 [batch] device copy of a ragged call's start positions
  std::vector<size_t> koff, voff, soff, zoff;
  // pipelined decode: cohort g holds sequences [g B, (g + 1) B), B = batch / n_passes.
  // A cohort between calls is parked in the looped block: its streams X, its
  // last sublayer output y and that site's maps (the pending write-back).
  size_t park_x = 0, park_y = 0, park_maps = 0;
  std::vector<int> pipe_next;   // pass the cohort runs at its next call; 0: no token in flight
  int pipe_enter = 0;           // cohort whose token enters next
  bool pipe_idle() const {
    for (size_t g = 0; g < pipe_next.size(); ++g)
      if (pipe_next[g] != 0) return false;
    return true;
  }
  void pipe_reset() {
    for (size_t g = 0; g < pipe_next.size(); ++g) pipe_next[g] = 0;
    pipe_enter = 0;
  }
  // shortest and longest length over sequences [s0, s0 + n)
  void lengths(int s0, int n, int* mn, int* mx) const {
    *mn = *mx = seq_len[s0];
    for (int i = s0 + 1; i < s0 + n; ++i) { *mn = std::min(*mn, seq_len[i]); *mx = std::max(*mx, seq_len[i]); }
  }
};

namespace {

struct WsLayout {
  size_t h, X, u, y, qkv, attn, inter, maps, lin, dec, dec_meta, wsplit, skinny, skinny_bytes, total;
  int wsplit_sites;   // mHC sites whose W split a call keeps (0: one scratch split per site visit)
};

WsLayout ws_layout(const loop_model* m, int batch, int max_tokens, int max_seq) {
  const loop_config& c = m->cfg;
  const size_t T = (size_t)max_tokens, C = c.hidden, es = m->es;
  WsLayout w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  w.h = take(T * C * es);
  w.X = take(T * 2 * C * es);
  w.u = take(T * C * es);
  w.y = take(T * C * es);
  w.qkv = take(T * m->qkv_rows() * es);
  w.attn = take(T * c.n_heads * c.head_dim * es);
  w.inter = take(T * c.ffn * es);
  w.maps = take(2 * T * 8 * sizeof(float));
  const size_t chunks = (T + LIN_CHUNK - 1) / LIN_CHUNK + (size_t)batch;
  w.lin = take(chunks * c.n_kv_heads * ((size_t)c.head_dim * c.head_dim + c.head_dim) * sizeof(float));
  // decode-attention partials: a call with B' <= batch sequences uses
  // B' * Hq * n_split(B') rows of d + 2 floats
  const int S_max = (max_seq + 63) / 64 * 64;
  size_t dec_rows = 0;
  for (int b = 1; b <= batch; ++b)
    dec_rows = std::max(dec_rows, (size_t)b * c.n_heads * lk::decode_max_splits(b, c.n_kv_heads, S_max, m->cu));
  // a ragged decode step (two sequences or more) splits stream-K: up to
  // decode_sk_slots partials per row, and the padded key prefix
  if (batch >= 2) dec_rows = std::max(dec_rows, (size_t)batch * c.n_heads * lk::decode_sk_slots(c.n_kv_heads, m->cu));
  w.dec = take(dec_rows * (c.head_dim + 2) * sizeof(float));
  w.dec_meta = take((size_t)(batch + 1) * sizeof(int32_t));
  // bf16 calls whose mHC sites run tiled keep each site's split of W (both
  // passes read it), plus one scratch split for a W seen beyond that count
  const bool site_splits = c.dtype == LOOP_BF16 && C % 512 == 0 && max_tokens >= lk::MHC_MFMA_MIN_T;
  w.wsplit_sites = site_splits ? 2 * (c.loop_end - c.loop_start) : 0;
  w.wsplit = take((size_t)(w.wsplit_sites + 1) * lk::MHC_WSPLIT_ROWS * 2 * C * sizeof(uint16_t));
  // split-K scratch of the decode-shaped GEMMs (the largest plan of the five projections)
  size_t sk = 0;
  if (c.dtype == LOOP_BF16 && max_tokens <= 64) {
    // the plan's partial size only grows with the token count (one or two blocks of 32)
    const int M = max_tokens;
    const lk::SkinnyPlan p[5] = {
        lk::skinny_plan(lk::EPI_QKV, M, m->qkv_rows(), C, 0, m->cu),
        lk::skinny_plan(lk::EPI_STORE, M, C, c.n_heads * c.head_dim, 0, m->cu),
        lk::skinny_plan(lk::EPI_SWIGLU, M, 2 * c.ffn, C, c.ffn, m->cu),
        lk::skinny_plan(lk::EPI_STORE, M, C, c.ffn, 0, m->cu),
        lk::skinny_plan(lk::EPI_F32, M, c.vocab, C, 0, m->cu)};
    for (const auto& q : p) sk = std::max(sk, q.bytes);
  }
  w.skinny = take(sk);
  w.skinny_bytes = sk;
  w.total = off;
  return w;
}

int check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return LOOP_OK;
  return lp_fail(LOOP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int noalloc_scratch(void** out) {
  int dev = -1;
  if (int r = check_hip(hipGetDevice(&dev), "hipGetDevice")) return r;
  if (dev < 0 || dev >= MAX_DEVICES)
    return lp_fail(LOOP_ERR_NO_DEVICE, "device %d outside the library's table of %d devices", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (int r = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)")) return r;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LOOP_OK;
}

}  // namespace

extern "C" {

const char* loop_status_string(int s) {
  switch (s) {
    case LOOP_OK: return "ok";
    case LOOP_ERR_INVALID_ARG: return "invalid argument";
    case LOOP_ERR_SHAPE: return "unsupported shape";
    case LOOP_ERR_ALIGN: return "misaligned pointer";
    case LOOP_ERR_CAPACITY: return "capacity exceeded";
    case LOOP_ERR_WORKSPACE: return "workspace too small";
    case LOOP_ERR_NO_DEVICE: return "no HIP device";
    case LOOP_ERR_HIP: return "HIP runtime error";
    case LOOP_ERR_DEVICE_FLAG: return "device-side input error";
    case LOOP_ERR_STATE: return "invalid state";
  }
  return "unknown status";
}

const char* loop_last_error(void) { return g_err.c_str(); }

int loop_model_create(const loop_config* cfg, const loop_weights* w, loop_model** out) {
  if (!cfg || !w || !out) return lp_fail(LOOP_ERR_INVALID_ARG, "null argument");
  *out = nullptr;
  const loop_config& c = *cfg;
  if (c.vocab <= 0 || c.hidden <= 0 || c.ffn <= 0 || c.n_heads <= 0 || c.n_kv_heads <= 0 ||
      c.head_dim <= 0 || c.n_layers <= 0)
    return lp_fail(LOOP_ERR_INVALID_ARG, "sizes must be positive");
  if (c.loop_start < 0 || c.loop_start > c.loop_end || c.loop_end > c.n_layers)
    return lp_fail(LOOP_ERR_INVALID_ARG, "loop range [%d, %d) not inside [0, %d]", c.loop_start, c.loop_end, c.n_layers);
  if (c.n_passes < 1) return lp_fail(LOOP_ERR_INVALID_ARG, "n_passes must be >= 1");
  if (c.sinkhorn_iters < 0 || c.attn_period < 1) return lp_fail(LOOP_ERR_INVALID_ARG, "sinkhorn_iters / attn_period");
  if (!(c.rms_eps > 0.f) || !(c.la_eps >= 0.f)) return lp_fail(LOOP_ERR_INVALID_ARG, "eps");
  if (c.dtype != LOOP_FP32 && c.dtype != LOOP_BF16) return lp_fail(LOOP_ERR_INVALID_ARG, "dtype");
  if (w->n_layers != c.n_layers || !w->layers) return lp_fail(LOOP_ERR_INVALID_ARG, "weights: layer count");
  if (c.n_heads % c.n_kv_heads || c.n_heads / c.n_kv_heads > 8)
    return lp_fail(LOOP_ERR_SHAPE, "n_heads must be a multiple of n_kv_heads, at most 8 per group");
  if (c.hidden % 8 || c.hidden > 4096) return lp_fail(LOOP_ERR_SHAPE, "hidden must be a multiple of 8, <= 4096");
  const int qkv_rows = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  if (c.dtype == LOOP_BF16) {
    if (c.head_dim != 128 && c.head_dim != 256) return lp_fail(LOOP_ERR_SHAPE, "bf16 needs head_dim 128 or 256");
    const int G = c.n_heads / c.n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && (G != 8 || c.head_dim != 128))
      return lp_fail(LOOP_ERR_SHAPE, "bf16 needs n_heads / n_kv_heads in 1, 2, 4 (or 8 with head_dim 128)");
    if (c.hidden % 256 || qkv_rows % 256 || c.vocab % 256 || (c.n_heads * c.head_dim) % 128 || c.ffn % 128)
      return lp_fail(LOOP_ERR_SHAPE, "bf16 GEMM tiles need hidden, qkv rows, vocab %% 256 == 0 and ffn %% 128 == 0");
    // The bf16 GEMM tiles address a weight matrix and 256 rows of an operand
    // with 32-bit element offsets, and 256 float32 logit rows with 32-bit
    // byte offsets.  Checked here, so that no call can fail on a shape after
    // it has launched part of a forward.
    const long lim = 1L << 31, C = c.hidden, F = c.ffn, Q = (long)c.n_heads * c.head_dim;
    if ((long)c.vocab * C >= lim || 2 * F * C >= lim || (long)qkv_rows * C >= lim || C * Q >= lim || C * F >= lim ||
        256L * std::max(F, Q) >= lim || 256L * c.vocab * 4 >= lim)
      return lp_fail(LOOP_ERR_SHAPE, "bf16 weight matrices need fewer than 2^31 elements and vocab < 2^21");
  } else {
    if (c.head_dim != 64 && c.head_dim != 128) return lp_fail(LOOP_ERR_SHAPE, "fp32 needs head_dim 64 or 128");
    if (c.ffn % 8 || (c.n_heads * c.head_dim) % 8) return lp_fail(LOOP_ERR_SHAPE, "fp32 widths must be multiples of 8");
  }
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) return lp_fail(LOOP_ERR_NO_DEVICE, "no HIP device");

  auto* m = new loop_model();
  m->cfg = c;
  m->es = c.dtype == LOOP_BF16 ? 2 : 4;
  m->embed = w->embed;
  m->final_norm = w->final_norm;
  m->head = w->head;
  m->layers.assign(w->layers, w->layers + c.n_layers);
  auto bad = [&](const char* what, int i) {
    delete m;
    return lp_fail(LOOP_ERR_INVALID_ARG, "weights: %s missing (layer %d)", what, i);
  };
  if (!m->embed || !m->final_norm || !m->head) return bad("embed/final_norm/head", -1);
  if (misaligned(m->embed) || misaligned(m->final_norm) || misaligned(m->head)) {
    delete m;
    return lp_fail(LOOP_ERR_ALIGN, "weights: global tensor not 16-byte aligned");
  }
  for (int i = 0; i < c.n_layers; ++i) {
    const loop_layer_weights& L = m->layers[i];
    if (!L.attn_norm || !L.ffn_norm || !L.qkv || !L.o || !L.gate_up || !L.down) return bad("layer tensor", i);
    const void* ps[6] = {L.attn_norm, L.ffn_norm, L.qkv, L.o, L.gate_up, L.down};
    for (const void* p : ps)
      if (misaligned(p)) { delete m; return lp_fail(LOOP_ERR_ALIGN, "weights: layer %d tensor not 16-byte aligned", i); }
    if (m->in_loop(i)) {
      for (int s = 0; s < 2; ++s) {
        if (!L.mhc_w[s] || !L.mhc_b[s]) return bad("mhc parameters", i);
        if (misaligned(L.mhc_w[s])) { delete m; return lp_fail(LOOP_ERR_ALIGN, "weights: mhc_w not 16-byte aligned"); }
      }
    }
  }
  // schedule: [0, ls) once, [ls, le) n_passes times, [le, L) once
  auto push = [&](int i, int p) {
    const int full = (i % c.attn_period) == c.attn_period - 1;
    m->sched.push_back({i, p, full, full ? m->n_full++ : m->n_lin++});
  };
  for (int i = 0; i < c.loop_start; ++i) push(i, 0);
  for (int p = 0; p < c.n_passes; ++p)
    for (int i = c.loop_start; i < c.loop_end; ++i) push(i, p);
  for (int i = c.loop_end; i < c.n_layers; ++i) push(i, 0);
  m->cu = lk::device_cu_count();
  if (m->cu <= 0) m->cu = 256;
  // set-up of loop_decode_step_noalloc: the static workspace's address on this device
  void* ws = nullptr;
  if (int r = noalloc_scratch(&ws)) {
    delete m;
    return r;
  }
  *out = m;
  return LOOP_OK;
}

int loop_model_destroy(loop_model* m) {
  delete m;
  return LOOP_OK;
}

int loop_model_schedule(const loop_model* m, int max, int* layer, int* pass, int* kind, int* slot, int* n) {
  if (!m || !n) return lp_fail(LOOP_ERR_INVALID_ARG, "null argument");
  *n = (int)m->sched.size();
  for (int e = 0; e < *n && e < max; ++e) {
    if (layer) layer[e] = m->sched[e].layer;
    if (pass) pass[e] = m->sched[e].pass;
    if (kind) kind[e] = m->sched[e].full;
    if (slot) slot[e] = m->sched[e].slot;
  }
  return LOOP_OK;
}

static void state_offsets(const loop_model* m, int batch, int max_seq, int n_pages, std::vector<size_t>* k,
                          std::vector<size_t>* v, std::vector<size_t>* s, std::vector<size_t>* z, size_t* total,
                          size_t* park = nullptr) {
  const loop_config& c = m->cfg;
  const size_t S_max = ((size_t)max_seq + 63) / 64 * 64;
  // contiguous: K [batch][Hkv][S_max][d] per slot; paged: a pool K [n_pages][Hkv][64][d]
  const size_t kv = (n_pages > 0 ? (size_t)n_pages * 64 : (size_t)batch * S_max) * c.n_kv_heads * c.head_dim * m->es;
  const size_t sb = (size_t)batch * c.n_kv_heads * c.head_dim * c.head_dim * sizeof(float);
  const size_t zb = (size_t)batch * c.n_kv_heads * c.head_dim * sizeof(float);
  size_t off = 256;
  for (int i = 0; i < m->n_full; ++i) {
    if (k) k->push_back(off);
    off += align256(kv);
    if (v) v->push_back(off);
    off += align256(kv);
  }
  for (int i = 0; i < m->n_lin; ++i) {
    if (s) s->push_back(off);
    off += align256(sb);
    if (z) z->push_back(off);
    off += align256(zb);
  }
  // parked cohorts of the pipelined decode: X [batch][2][C], y [batch][C], maps [batch][8] fp32
  const size_t C = c.hidden;
  if (park) park[0] = off;
  off += align256((size_t)batch * 2 * C * m->es);
  if (park) park[1] = off;
  off += align256((size_t)batch * C * m->es);
  if (park) park[2] = off;
  off += align256((size_t)batch * 8 * sizeof(float));
  // start positions of a ragged call, int32 [batch]
  if (park) park[3] = off;
  off += align256((size_t)batch * sizeof(int32_t));
  *total = off;
}

int loop_state_bytes(const loop_model* m, int batch, int max_seq, size_t* bytes) {
  if (!m || !bytes) return lp_fail(LOOP_ERR_INVALID_ARG, "null argument");
  if (batch <= 0 || max_seq <= 0) return lp_fail(LOOP_ERR_INVALID_ARG, "batch and max_seq must be positive");
  state_offsets(m, batch, max_seq, 0, nullptr, nullptr, nullptr, nullptr, bytes);
  return LOOP_OK;
}

int loop_workspace_bytes(const loop_model* m, int batch, int max_tokens, int max_seq, size_t* bytes) {
  if (!m || !bytes) return lp_fail(LOOP_ERR_INVALID_ARG, "null argument");
  if (batch <= 0 || max_tokens <= 0 || max_seq <= 0) return lp_fail(LOOP_ERR_INVALID_ARG, "sizes must be positive");
  *bytes = ws_layout(m, batch, max_tokens, max_seq).total;
  return LOOP_OK;
}

// Largest cache length of a paged state: the prefill attention keeps the page
// numbers of a workgroup's tiles (up to 8,192) in LDS next to its ring.
constexpr int PAGED_MAX_SEQ = 8192 * 64;

int loop_state_bytes_paged(const loop_model* m, int batch, int max_seq, int n_pages, size_t* bytes) {
  if (!m || !bytes) return lp_fail(LOOP_ERR_INVALID_ARG, "null argument");
  if (batch <= 0 || max_seq <= 0 || n_pages <= 0)
    return lp_fail(LOOP_ERR_INVALID_ARG, "batch, max_seq and n_pages must be positive");
  state_offsets(m, batch, max_seq, n_pages, nullptr, nullptr, nullptr, nullptr, bytes);
  return LOOP_OK;
}

static int state_create(const loop_model* m, void* state_dev, size_t bytes, int batch, int max_seq, int n_pages,
                        const int32_t* table, loop_state** out) {
  if (!m || !state_dev || !out) return lp_fail(LOOP_ERR_INVALID_ARG, "null argument");
  *out = nullptr;
  if (batch <= 0 || max_seq <= 0) return lp_fail(LOOP_ERR_INVALID_ARG, "batch and max_seq must be positive");
  if (misaligned(state_dev)) return lp_fail(LOOP_ERR_ALIGN, "state not 16-byte aligned");
  if (n_pages > 0) {
    if (!table) return lp_fail(LOOP_ERR_INVALID_ARG, "null block table");
    if ((uintptr_t)table % 4) return lp_fail(LOOP_ERR_ALIGN, "block table not 4-byte aligned");
    if (max_seq > PAGED_MAX_SEQ) return lp_fail(LOOP_ERR_CAPACITY, "paged state: max_seq %d above %d", max_seq, PAGED_MAX_SEQ);
  }
  auto* st = new loop_state();
  size_t need = 0, park[4] = {0, 0, 0, 0};
  state_offsets(m, batch, max_seq, n_pages, &st->koff, &st->voff, &st->soff, &st->zoff, &need, park);
  if (bytes < need) {
    delete st;
    return lp_fail(LOOP_ERR_CAPACITY, "state has %zu bytes, needs %zu", bytes, need);
  }
  st->m = m;
  st->base = (char*)state_dev;
  st->bytes = bytes;
  st->batch = batch;
  st->max_seq = max_seq;
  st->S_max = (max_seq + 63) / 64 * 64;
  st->seq_len.assign(batch, 0);
  st->park_x = park[0];
  st->park_y = park[1];
  st->park_maps = park[2];
  st->pos_off = park[3];
  st->pipe_next.assign(m->cfg.n_passes, 0);
  if (n_pages > 0) {
    st->n_pages = n_pages;
    st->table = table;
    st->table_stride = (max_seq + 63) / 64;
  }
  *out = st;
  return LOOP_OK;
}

int loop_state_create(const loop_model* m, void* state_dev, size_t bytes, int batch, int max_seq, loop_state** out) {
  return state_create(m, state_dev, bytes, batch, max_seq, 0, nullptr, out);
}

int loop_state_create_paged(const loop_model* m, void* state_dev, size_t bytes, int batch, int max_seq, int n_pages,
                            const int32_t* block_table_dev, loop_state** out) {
  if (n_pages <= 0) return lp_fail(LOOP_ERR_INVALID_ARG, "n_pages must be positive");
  return state_create(m, state_dev, bytes, batch, max_seq, n_pages, block_table_dev, out);
}

int loop_state_destroy(loop_state* st) {
  delete st;
  return LOOP_OK;
}

int loop_state_length(const loop_state* st, int* length) {
  if (!st || !length) return lp_fail(LOOP_ERR_INVALID_ARG, "null argument");
  int mx;
  st->lengths(0, st->batch, length, &mx);
  return LOOP_OK;
}

int loop_state_set_length(loop_state* st, int length) {
  if (!st) return lp_fail(LOOP_ERR_INVALID_ARG, "null argument");
  if (length < 0 || length > st->max_seq) return lp_fail(LOOP_ERR_CAPACITY, "length %d outside [0, %d]", length, st->max_seq);
  st->seq_len.assign(st->batch, length);
  st->pipe_reset();
  return LOOP_OK;
}

int loop_state_seq_length(const loop_state* st, int seq, int* length) {
  if (!st || !length) return lp_fail(LOOP_ERR_INVALID_ARG, "null argument");
  if (seq < 0 || seq >= st->batch) return lp_fail(LOOP_ERR_INVALID_ARG, "sequence %d outside [0, %d)", seq, st->batch);
  *length = st->seq_len[seq];
  return LOOP_OK;
}

int loop_state_set_seq_length(loop_state* st, int seq, int length) {
  if (!st) return lp_fail(LOOP_ERR_INVALID_ARG, "null argument");
  if (seq < 0 || seq >= st->batch) return lp_fail(LOOP_ERR_INVALID_ARG, "sequence %d outside [0, %d)", seq, st->batch);
  if (length < 0 || length > st->max_seq) return lp_fail(LOOP_ERR_CAPACITY, "length %d outside [0, %d]", length, st->max_seq);
  st->seq_len[seq] = length;
  st->pipe_reset();
  return LOOP_OK;
}

int loop_state_region(const loop_state* st, int kind, int slot, void** ptr, size_t* bytes) {
  if (!st || !ptr) return lp_fail(LOOP_ERR_INVALID_ARG, "null argument");
  const loop_model* m = st->m;
  const loop_config& c = m->cfg;
  size_t off = 0, sz = 0;
  const size_t kv = (st->table ? (size_t)st->n_pages * 64 : (size_t)st->batch * st->S_max) * c.n_kv_heads *
                    c.head_dim * m->es;
  switch (kind) {
    case 0: case 1:
      if (slot < 0 || slot >= m->n_full) return lp_fail(LOOP_ERR_INVALID_ARG, "full slot %d out of range", slot);
      off = kind == 0 ? st->koff[slot] : st->voff[slot];
      sz = kv;
      break;
    case 2: case 3:
      if (slot < 0 || slot >= m->n_lin) return lp_fail(LOOP_ERR_INVALID_ARG, "linear slot %d out of range", slot);
      off = kind == 2 ? st->soff[slot] : st->zoff[slot];
      sz = (size_t)st->batch * c.n_kv_heads * c.head_dim * (kind == 2 ? c.head_dim : 1) * sizeof(float);
      break;
    case 4:
      off = 0;
      sz = 256;
      break;
    default:
      return lp_fail(LOOP_ERR_INVALID_ARG, "region kind %d", kind);
  }
  *ptr = st->base + off;
  if (bytes) *bytes = sz;
  return LOOP_OK;
}

int loop_state_check(loop_state* st, void* stream) {
  if (!st) return lp_fail(LOOP_ERR_INVALID_ARG, "null argument");
  hipStream_t s = (hipStream_t)stream;
  uint32_t word = 0;
  int r = check_hip(hipMemcpyAsync(&word, st->base, sizeof word, hipMemcpyDeviceToHost, s), "read error word");
  if (r) return r;
  r = check_hip(hipStreamSynchronize(s), "synchronize");
  if (r) return r;
  if (word) {
    r = check_hip(hipMemsetAsync(st->base, 0, sizeof word, s), "clear error word");
    if (r) return r;
    r = check_hip(hipStreamSynchronize(s), "synchronize");
    if (r) return r;
    return lp_fail(LOOP_ERR_DEVICE_FLAG, "device flagged input error 0x%x (token id out of range)", word);
  }
  return LOOP_OK;
}

}  // extern "C"

namespace {

#define LAUNCH(call, what)                                   \
  do {                                                       \
    hipError_t e_ = (call);                                  \
    if (e_ != hipSuccess) return check_hip(e_, what);        \
  } while (0)

// Runs sequences [seq0, seq0 + B) of the state, S new positions each.  A
// decode step takes every sequence at its own length (ragged rows read their
// start positions from the state's device copy); a prefill starts the rows at
// 0, or with LOOP_CONTINUE at their common length.
int forward(loop_model* m, loop_state* st, void* workspace, size_t ws_bytes, int seq0, const int32_t* tokens,
            const void* embeds, int B, int S, unsigned flags, void* out, hipStream_t s, bool decode) {
  const loop_config& c = m->cfg;
  if (!st || st->m != m) return lp_fail(LOOP_ERR_STATE, "state does not belong to this model");
  if (!workspace || !out || (!tokens && !embeds)) return lp_fail(LOOP_ERR_INVALID_ARG, "null argument");
  if (B <= 0 || S <= 0) return lp_fail(LOOP_ERR_INVALID_ARG, "B and S must be positive");
  if (misaligned(workspace) || misaligned(out) || misaligned(embeds)) return lp_fail(LOOP_ERR_ALIGN, "misaligned buffer");
  if (seq0 < 0 || seq0 >= st->batch) return lp_fail(LOOP_ERR_INVALID_ARG, "first sequence %d outside [0, %d)", seq0, st->batch);
  if (B > st->batch - seq0)
    return lp_fail(LOOP_ERR_CAPACITY, "sequences [%d, %d) exceed the state's %d", seq0, seq0 + B, st->batch);
  if (!st->pipe_idle())
    return lp_fail(LOOP_ERR_STATE, "pipelined decode in progress (a cohort has a token in flight)");
  int len_min, len_max;
  st->lengths(seq0, B, &len_min, &len_max);
  if (decode && len_min == 0) return lp_fail(LOOP_ERR_STATE, "decode before prefill");
  if (!decode && (flags & LOOP_CONTINUE) && len_min != len_max)
    return lp_fail(LOOP_ERR_STATE, "continued prefill over sequences of different lengths (%d..%d)", len_min, len_max);
  // pos0: the (largest) first new position; ragged decode rows read their own
  const int pos0 = (decode || (flags & LOOP_CONTINUE)) ? len_max : 0;
  const bool ragged = decode && len_min != len_max;
  // lengths far apart (the shortest under 7/8 of the longest): the bf16 decode
  // attention splits the keys of all sequences stream-K
  const bool ragged_sk = ragged && c.dtype == LOOP_BF16 && (long)(len_max - len_min) * 8 > len_max;
  if ((long)pos0 + S > st->max_seq)
    return lp_fail(LOOP_ERR_CAPACITY, "positions %d + %d exceed max_seq %d", pos0, S, st->max_seq);
  const int T = B * S;
  const WsLayout L = ws_layout(m, B, T, st->max_seq);
  if (ws_bytes < L.total) return lp_fail(LOOP_ERR_WORKSPACE, "workspace %zu bytes, needs %zu", ws_bytes, L.total);

  char* ws = (char*)workspace;
  void* h = ws + L.h;
  void* X = ws + L.X;
  void* u = ws + L.u;
  void* y = ws + L.y;
  void* qkv = ws + L.qkv;
  void* attn = ws + L.attn;
  void* inter = ws + L.inter;
  float* maps[2] = {(float*)(ws + L.maps), (float*)(ws + L.maps) + (size_t)T * 8};
  float* lin_scr = (float*)(ws + L.lin);
  float* dec_part = (float*)(ws + L.dec);
  const int dt = c.dtype == LOOP_BF16 ? lk::DT_BF16 : lk::DT_F32;
  const int C = c.hidden, Hq = c.n_heads, Hkv = c.n_kv_heads, d = c.head_dim;
  const int qkv_rows = m->qkv_rows();
  const int mhc_grid = T < 2 * m->cu ? T : 2 * m->cu;
  // per-sequence slices of the slots: the kernels index sequences from the base
  const size_t kv_skip = st->kv_seq_off(seq0, (size_t)Hkv * st->S_max * d * m->es);
  const lk::KvPages pages = st->pages(seq0);
  const size_t s_skip = (size_t)seq0 * Hkv * d * d, z_skip = (size_t)seq0 * Hkv * d;
  const int* pos_dev = nullptr;
  if (ragged) {
    int32_t* p = (int32_t*)(st->base + st->pos_off) + seq0;
    LAUNCH(lk::set_i32(p, st->seq_len.data() + seq0, B, s), "positions");
    pos_dev = p;
  }
  lk::StreamKPlan sk{};
  const int32_t* sk_pref = nullptr;
  if (ragged_sk) {
    std::vector<int32_t> pref(B + 1, 0);
    for (int b = 0; b < B; ++b) pref[b + 1] = pref[b] + (st->seq_len[seq0 + b] + S + 63) / 64 * 64;
    sk = lk::decode_plan_sk(pref[B], Hkv, m->cu);
    int32_t* p = (int32_t*)(ws + L.dec_meta);
    LAUNCH(lk::set_i32(p, pref.data(), B + 1, s), "key prefix");
    sk_pref = p;
  }

  // embedding
  if (tokens) {
    LAUNCH(lk::embed(dt, tokens, m->embed, c.vocab, C, T, h, (uint32_t*)st->base, s), "embed");
  } else {
    LAUNCH(hipMemcpyAsync(h, embeds, (size_t)T * C * m->es, hipMemcpyDeviceToDevice, s), "copy embeds");
  }

  // Decode-shaped o and down projections leave their split-K partials in the
  // workspace; the norm or mHC kernel that consumes y sums them (ypend).
  lk::YPart ypend{};
  auto norm = [&](const void* yin, const float* gamma) {
    lk::NormArgs a{};
    a.dt = dt; a.T = T; a.C = C; a.y = yin; a.h = h; a.gamma = gamma; a.u = u; a.eps = c.rms_eps;
    if (yin) a.yp = ypend;
    ypend = lk::YPart{};
    return lk::add_rmsnorm(a, s);
  };
  int mp = 0;   // maps[mp] holds the maps of the current mHC site
  std::vector<const float*> split_w;   // W of the sites whose split is in the workspace, by slot
  auto mhc = [&](int mode, const void* yin, const float* w, const float* b, const float* gamma) {
    lk::MhcArgs a{};
    a.dt = dt; a.mode = mode; a.T = T; a.C = C; a.iters = c.sinkhorn_iters; a.eps = c.rms_eps;
    a.y = yin; a.h = h; a.X = X;
    if (yin) a.yp = ypend;
    ypend = lk::YPart{};
    a.maps_in = maps[mp];
    a.maps_out = maps[mp ^ 1];
    a.w = w; a.b = b; a.gamma = gamma; a.u = u; a.grid = mhc_grid;
    a.wsplit = (lk::bf16_t*)(ws + L.wsplit);
    if (L.wsplit_sites > 0 && w && mode != lk::MHC_EXIT) {
      // the second pass (and a site met again) reuses the split made at the first visit
      size_t k = 0;
      while (k < split_w.size() && split_w[k] != w) ++k;
      if (k < split_w.size()) a.wsplit_ready = 1;
      else if (k < (size_t)L.wsplit_sites) split_w.push_back(w);
      a.wsplit += k * (size_t)lk::MHC_WSPLIT_ROWS * 2 * C;
    }
    hipError_t e = lk::mhc(a, s);
    if (mode != lk::MHC_EXIT) mp ^= 1;
    return e;
  };
  // decode-shaped GEMMs split K over workgroups when the workspace holds the scratch
  auto run_gemm = [&](lk::GemmArgs g, bool may_defer = false) {
    g.ksplit = 1;
    if (g.dt == lk::DT_BF16 && g.M <= 64) {
      const lk::SkinnyPlan p = lk::skinny_plan(g.epi, g.M, g.N, g.K, g.F, m->cu);
      if (p.ksplit > 1 && p.bytes <= L.skinny_bytes) {
        g.ksplit = p.ksplit;
        g.part = (float*)(ws + L.skinny);
        if (may_defer && g.epi == lk::EPI_STORE) {
          g.defer_reduce = 1;
          ypend = lk::YPart{g.part, p.ksplit, 32 * p.rb, 32 * p.tb};
        }
      }
    }
    return lk::gemm(g, s);
  };
  auto gemm = [&](int epi, const void* A, long lda, int M, const void* Bw, int N, int K, void* Cout, long ldc) {
    lk::GemmArgs g{};
    g.dt = dt; g.epi = epi; g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.B = Bw; g.ldb = K; g.C = Cout; g.ldc = ldc;
    return g;
  };

  const auto& sched = m->sched;
  const int E = (int)sched.size();
  {
    const loop_layer_weights& L0 = m->layers[sched[0].layer];
    if (m->in_loop(sched[0].layer)) {
      LAUNCH(mhc(lk::MHC_ENTER, nullptr, L0.mhc_w[0], L0.mhc_b[0], L0.attn_norm), "mhc enter");
    } else {
      LAUNCH(norm(nullptr, L0.attn_norm), "rmsnorm");
    }
  }
  for (int e = 0; e < E; ++e) {
    const Exec& ex = sched[e];
    const loop_layer_weights& W = m->layers[ex.layer];
    const bool looped = m->in_loop(ex.layer);
    // ---- attention sublayer
    if (ex.full) {
      lk::GemmArgs g = gemm(lk::EPI_QKV, u, C, T, W.qkv, qkv_rows, C, qkv, qkv_rows);
      g.q_cols = Hq * d; g.n_kv = Hkv; g.head_dim = d;
      g.kcache = st->base + st->koff[ex.slot] + kv_skip;
      g.vcache = st->base + st->voff[ex.slot] + kv_skip;
      g.S_call = S; g.pos0 = pos0; g.S_max = st->S_max; g.pos_dev = pos_dev; g.pages = pages;
      if (pages.table && dt == lk::DT_BF16 && T > 64) {
        // the 256-row tile GEMM stores contiguous caches only: plain rows, then the pages
        g.epi = lk::EPI_STORE;
        LAUNCH(run_gemm(g), "qkv gemm");
        LAUNCH(lk::kv_scatter(dt, qkv, qkv_rows, Hq * d, B, S, pos0, pos_dev, Hkv, d, g.kcache, g.vcache, st->S_max,
                              pages, s),
               "kv scatter");
      } else {
        LAUNCH(run_gemm(g), "qkv gemm");
      }
      lk::AttnArgs a{};
      a.dt = dt; a.B = B; a.S_call = S; a.pos0 = pos0; a.S_max = st->S_max; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
      a.pos_dev = pos_dev; a.pages = pages;
      a.q = qkv; a.ldq = qkv_rows; a.kcache = g.kcache; a.vcache = g.vcache; a.out = attn; a.ldo = Hq * d;
      if (decode && sk_pref) {
        a.part = dec_part;
        LAUNCH(lk::attn_decode_sk(a, sk_pref, sk, s), "decode attention (stream-K)");
      } else if (decode && dt == lk::DT_BF16) {
        const lk::DecodePlan dp = lk::decode_plan(B, Hkv, pos0 + S, m->cu);
        a.part = dec_part; a.split_len = dp.split_len; a.n_split = dp.n_split;
        LAUNCH(lk::attn_decode(a, s), "decode attention");
      } else {
        LAUNCH(lk::attn_prefill(a, s), "prefill attention");
      }
    } else {
      lk::GemmArgs g = gemm(lk::EPI_STORE, u, C, T, W.qkv, qkv_rows, C, qkv, qkv_rows);
      LAUNCH(run_gemm(g, decode && S <= 16), "qkv gemm");
      lk::LinArgs a{};
      a.qp = ypend;                    // set when the projection left partials
      ypend = lk::YPart{};
      a.dt = dt; a.B = B; a.S_call = S; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.eps = c.la_eps;
      a.qkv = qkv; a.ld = qkv_rows;
      a.S = (float*)(st->base + st->soff[ex.slot]) + s_skip;
      a.z = (float*)(st->base + st->zoff[ex.slot]) + z_skip;
      a.init_zero = pos0 == 0;
      a.out = attn; a.ldo = Hq * d; a.scratch = lin_scr; a.chunk = LIN_CHUNK;
      if (S <= 16) { LAUNCH(lk::lin_decode(a, s), "linear attention (recurrent)"); }
      else { LAUNCH(lk::lin_prefill(a, s), "linear attention (chunked)"); }
    }
    LAUNCH(run_gemm(gemm(lk::EPI_STORE, attn, Hq * d, T, W.o, C, Hq * d, y, C), decode), "o gemm");
    // ---- attention -> FFN transition
    if (looped) {
      LAUNCH(mhc(lk::MHC_MID, y, W.mhc_w[1], W.mhc_b[1], W.ffn_norm), "mhc");
    } else {
      LAUNCH(norm(y, W.ffn_norm), "add+rmsnorm");
    }
    // ---- FFN sublayer
    {
      lk::GemmArgs g = gemm(lk::EPI_SWIGLU, u, C, T, W.gate_up, 2 * c.ffn, C, inter, c.ffn);
      g.F = c.ffn;
      LAUNCH(run_gemm(g), "gate/up gemm");
    }
    LAUNCH(run_gemm(gemm(lk::EPI_STORE, inter, c.ffn, T, W.down, C, c.ffn, y, C), decode), "down gemm");
    // ---- transition to the next execution (or the final norm)
    const bool has_next = e + 1 < E;
    const loop_layer_weights* Wn = has_next ? &m->layers[sched[e + 1].layer] : nullptr;
    const bool next_looped = has_next && m->in_loop(sched[e + 1].layer);
    const float* gamma_next = has_next ? Wn->attn_norm : m->final_norm;
    if (looped) {
      if (next_looped) {
        LAUNCH(mhc(lk::MHC_MID, y, Wn->mhc_w[0], Wn->mhc_b[0], gamma_next), "mhc");
      } else {
        LAUNCH(mhc(lk::MHC_EXIT, y, nullptr, nullptr, gamma_next), "mhc exit");
      }
    } else if (next_looped) {
      LAUNCH(mhc(lk::MHC_ENTER, y, Wn->mhc_w[0], Wn->mhc_b[0], gamma_next), "mhc enter");
    } else {
      LAUNCH(norm(y, gamma_next), "add+rmsnorm");
    }
  }
  // ---- output
  if (flags & LOOP_HIDDEN_OUT) {
    LAUNCH(hipMemcpyAsync(out, h, (size_t)T * C * m->es, hipMemcpyDeviceToDevice, s), "copy hidden");
  } else if (flags & LOOP_ALL_LOGITS) {
    LAUNCH(run_gemm(gemm(lk::EPI_F32, u, C, T, m->head, c.vocab, C, out, c.vocab)), "head gemm");
  } else {
    // the last position of every sequence: with S > 1 its B rows are gathered
    // into one contiguous block first (y is free once the final norm has read
    // it), so the head reads rows of stride C whatever S is
    const void* last = u;
    if (S > 1) {
      LAUNCH(hipMemcpy2DAsync(y, (size_t)C * m->es, (const char*)u + (size_t)(S - 1) * C * m->es,
                              (size_t)S * C * m->es, (size_t)C * m->es, B, hipMemcpyDeviceToDevice, s),
             "gather last rows");
      last = y;
    }
    LAUNCH(run_gemm(gemm(lk::EPI_F32, last, C, B, m->head, c.vocab, C, out, c.vocab)), "head gemm");
  }
  for (int b = seq0; b < seq0 + B; ++b) st->seq_len[b] = (decode ? st->seq_len[b] : pos0) + S;
  return LOOP_OK;
}

// Decode with the passes of the looped block co-scheduled over n_passes
// cohorts (cohort g = sequences [g B, (g + 1) B)).  A token enters its cohort
// with the layers before the block and pass 1, advances one pass per call
// (parked in the block between calls), and leaves after pass P with the
// layers after the block and the head.  Every call runs each stored layer of
// the block once for all cohorts' rows, so its weights are read once for up
// to P tokens' passes; attention and linear attention run per cohort on the
// cohort's own (layer, pass) slot and position.  Rows of a cohort with no
// token in flight go through the shared projections and stream kernels as
// don't-care rows whose results nothing reads.
int decode_pipelined(loop_model* m, loop_state* st, void* workspace, size_t ws_bytes, const int32_t* tokens, int B,
                     float* logits, int* info, hipStream_t s) {
  const loop_config& c = m->cfg;
  const int G = c.n_passes;
  if (!st || st->m != m) return lp_fail(LOOP_ERR_STATE, "state does not belong to this model");
  if (!workspace || !info) return lp_fail(LOOP_ERR_INVALID_ARG, "null argument");
  if (B <= 0 || st->batch != G * B)
    return lp_fail(LOOP_ERR_SHAPE, "pipelined decode needs a state of n_passes x cohort sequences (%d x %d != %d)", G,
                   B, st->batch);
  if (misaligned(workspace) || misaligned(logits)) return lp_fail(LOOP_ERR_ALIGN, "misaligned buffer");
  info[0] = info[1] = -1;
  std::vector<int> pass(G, 0);     // pass each cohort runs in this call (0: none)
  for (int g = 0; g < G; ++g)
    if (st->pipe_next[g] >= 2) pass[g] = st->pipe_next[g];
  int e = -1;
  if (tokens) {
    e = st->pipe_enter;
    if (st->pipe_next[e] != 0) return lp_fail(LOOP_ERR_STATE, "cohort %d still has a token in flight", e);
    int mn, mx;
    st->lengths(e * B, B, &mn, &mx);
    if (mn == 0) return lp_fail(LOOP_ERR_STATE, "decode before prefill");
    if (mn != mx) return lp_fail(LOOP_ERR_STATE, "cohort %d holds sequences of different lengths (%d..%d)", e, mn, mx);
    pass[e] = 1;
  }
  int f = -1;
  for (int g = 0; g < G; ++g)
    if (pass[g] == G) f = g;
  bool any = false;
  for (int g = 0; g < G; ++g) any = any || pass[g] > 0;
  if (!any) return lp_fail(LOOP_ERR_STATE, "no token to decode (no cohort in flight and no tokens given)");
  if (f >= 0 && !logits) return lp_fail(LOOP_ERR_INVALID_ARG, "null logits");
  for (int g = 0; g < G; ++g)
    if (pass[g] && st->seq_len[g * B] >= st->max_seq)
      return lp_fail(LOOP_ERR_CAPACITY, "cohort %d is at max_seq %d", g, st->max_seq);
  const int T = G * B;
  const WsLayout L = ws_layout(m, T, T, st->max_seq);
  if (ws_bytes < L.total) return lp_fail(LOOP_ERR_WORKSPACE, "workspace %zu bytes, needs %zu", ws_bytes, L.total);

  char* ws = (char*)workspace;
  const size_t es = m->es;
  const int dt = c.dtype == LOOP_BF16 ? lk::DT_BF16 : lk::DT_F32;
  const int C = c.hidden, Hq = c.n_heads, Hkv = c.n_kv_heads, d = c.head_dim, F = c.ffn;
  const int qkv_rows = m->qkv_rows();
  char* h = ws + L.h;
  char* u = ws + L.u;
  char* y = ws + L.y;
  char* qkv = ws + L.qkv;
  char* attn = ws + L.attn;
  char* inter = ws + L.inter;
  float* maps[2] = {(float*)(ws + L.maps), (float*)(ws + L.maps) + (size_t)T * 8};
  float* lin_scr = (float*)(ws + L.lin);
  float* dec_part = (float*)(ws + L.dec);
  char* X = st->base + st->park_x;
  char* parkY = st->base + st->park_y;
  float* parkM = (float*)(st->base + st->park_maps);
  const int ls = c.loop_start, le = c.loop_end, nl = le - ls;
  auto rows = [&](char* p, int r, size_t width) { return p + (size_t)r * width * es; };

  lk::YPart ypend{};
  auto run_gemm = [&](lk::GemmArgs g, bool may_defer) {
    g.ksplit = 1;
    if (g.dt == lk::DT_BF16 && g.M <= 64) {
      const lk::SkinnyPlan p = lk::skinny_plan(g.epi, g.M, g.N, g.K, g.F, m->cu);
      if (p.ksplit > 1 && p.bytes <= L.skinny_bytes) {
        g.ksplit = p.ksplit;
        g.part = (float*)(ws + L.skinny);
        if (may_defer && g.epi == lk::EPI_STORE) {
          g.defer_reduce = 1;
          ypend = lk::YPart{g.part, p.ksplit, 32 * p.rb, 32 * p.tb};
        }
      }
    }
    return lk::gemm(g, s);
  };
  auto gemm = [&](int epi, const void* A, long lda, int M, const void* Bw, int N, int K, void* Cout, long ldc) {
    lk::GemmArgs g{};
    g.dt = dt; g.epi = epi; g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.B = Bw; g.ldb = K; g.C = Cout; g.ldc = ldc;
    return g;
  };
  // rows [r0, r0 + n): h <- h + y (y may be null), u <- RMSNorm(h; gamma)
  auto norm = [&](int r0, int n, bool with_y, const float* gamma) {
    lk::NormArgs a{};
    a.dt = dt; a.T = n; a.C = C; a.y = with_y ? rows(y, r0, C) : nullptr; a.h = rows(h, r0, C); a.gamma = gamma;
    a.u = rows(u, r0, C); a.eps = c.rms_eps;
    if (with_y) a.yp = ypend;
    ypend = lk::YPart{};
    return lk::add_rmsnorm(a, s);
  };
  // one mHC transition on rows [r0, r0 + n)
  auto mhc = [&](int mode, int r0, int n, const void* yin, bool use_ypend, const float* mi, float* mo,
                 const float* w, const float* b, const float* gamma) {
    lk::MhcArgs a{};
    a.dt = dt; a.mode = mode; a.T = n; a.C = C; a.iters = c.sinkhorn_iters; a.eps = c.rms_eps;
    a.y = yin; a.h = rows(h, r0, C); a.X = rows(X, r0, 2 * C);
    if (use_ypend) a.yp = ypend;
    ypend = lk::YPart{};
    a.maps_in = mi ? mi + (size_t)r0 * 8 : nullptr;
    a.maps_out = mo ? mo + (size_t)r0 * 8 : nullptr;
    a.w = w; a.b = b; a.gamma = gamma; a.u = rows(u, r0, C);
    a.grid = n < 2 * m->cu ? n : 2 * m->cu;
    a.wsplit = (lk::bf16_t*)(ws + L.wsplit);
    return lk::mhc(a, s);
  };
  // attention sublayer of stored layer `layer` on rows [r0, r0 + n); cohorts in
  // `coh` (each a block of B rows inside the range) run their own execution
  // `ex_of(g)` at the cohort's common length; the O projection leaves y (deferred
  // when `defer_o`)
  auto attention = [&](int layer, int r0, int n, const std::vector<int>& coh, const std::vector<const Exec*>& exs,
                       bool defer_o) -> int {
    const loop_layer_weights& W = m->layers[layer];
    const bool full = exs[0]->full;
    const bool fused = full && (int)coh.size() == 1 && n == B;
    if (fused) {
      // one cohort: K and V go into its slot from the projection's epilogue
      const int g = coh[0];
      lk::GemmArgs q = gemm(lk::EPI_QKV, rows(u, r0, C), C, n, W.qkv, qkv_rows, C, rows(qkv, r0, qkv_rows), qkv_rows);
      q.q_cols = Hq * d; q.n_kv = Hkv; q.head_dim = d;
      q.kcache = st->base + st->koff[exs[0]->slot] + st->kv_seq_off(g * B, (size_t)Hkv * st->S_max * d * es);
      q.vcache = st->base + st->voff[exs[0]->slot] + st->kv_seq_off(g * B, (size_t)Hkv * d * st->S_max * es);
      q.S_call = 1; q.pos0 = st->seq_len[g * B]; q.S_max = st->S_max; q.pages = st->pages(g * B);
      LAUNCH(run_gemm(q, false), "qkv gemm");
    } else {
      LAUNCH(run_gemm(gemm(lk::EPI_STORE, rows(u, r0, C), C, n, W.qkv, qkv_rows, C, rows(qkv, r0, qkv_rows),
                           qkv_rows), false), "qkv gemm");
    }
    for (size_t i = 0; i < coh.size(); ++i) {
      const int g = coh[i];
      const Exec& ex = *exs[i];
      const int pos = st->seq_len[g * B];
      char* qrow = rows(qkv, g * B, qkv_rows);
      if (full) {
        char* kc = st->base + st->koff[ex.slot] + st->kv_seq_off(g * B, (size_t)Hkv * st->S_max * d * es);
        char* vc = st->base + st->voff[ex.slot] + st->kv_seq_off(g * B, (size_t)Hkv * d * st->S_max * es);
        const lk::KvPages pg = st->pages(g * B);
        if (!fused)
          LAUNCH(lk::kv_append(dt, qrow, qkv_rows, Hq * d, B, Hkv, d, kc, vc, st->S_max, pos, pg, s), "kv append");
        lk::AttnArgs a{};
        a.dt = dt; a.B = B; a.S_call = 1; a.pos0 = pos; a.S_max = st->S_max; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
        a.pages = pg;
        a.q = qrow; a.ldq = qkv_rows; a.kcache = kc; a.vcache = vc; a.out = rows(attn, g * B, Hq * d);
        a.ldo = Hq * d;
        if (dt == lk::DT_BF16) {
          const lk::DecodePlan dp = lk::decode_plan(B, Hkv, pos + 1, m->cu);
          a.part = dec_part; a.split_len = dp.split_len; a.n_split = dp.n_split;
          LAUNCH(lk::attn_decode(a, s), "decode attention");
        } else {
          LAUNCH(lk::attn_prefill(a, s), "attention");
        }
      } else {
        lk::LinArgs a{};
        a.dt = dt; a.B = B; a.S_call = 1; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.eps = c.la_eps;
        a.qkv = qrow; a.ld = qkv_rows;
        a.S = (float*)(st->base + st->soff[ex.slot]) + (size_t)g * B * Hkv * d * d;
        a.z = (float*)(st->base + st->zoff[ex.slot]) + (size_t)g * B * Hkv * d;
        a.init_zero = pos == 0;
        a.out = rows(attn, g * B, Hq * d); a.ldo = Hq * d; a.scratch = lin_scr; a.chunk = LIN_CHUNK;
        LAUNCH(lk::lin_decode(a, s), "linear attention (recurrent)");
      }
    }
    LAUNCH(run_gemm(gemm(lk::EPI_STORE, rows(attn, r0, Hq * d), Hq * d, n, W.o, C, Hq * d, rows(y, r0, C), C),
                    defer_o), "o gemm");
    return LOOP_OK;
  };
  auto ffn = [&](int layer, int r0, int n, bool defer_down) -> int {
    const loop_layer_weights& W = m->layers[layer];
    lk::GemmArgs g = gemm(lk::EPI_SWIGLU, rows(u, r0, C), C, n, W.gate_up, 2 * F, C, rows(inter, r0, F), F);
    g.F = F;
    LAUNCH(run_gemm(g, false), "gate/up gemm");
    LAUNCH(run_gemm(gemm(lk::EPI_STORE, rows(inter, r0, F), F, n, W.down, C, F, rows(y, r0, C), C), defer_down),
           "down gemm");
    return LOOP_OK;
  };
  // the plain (outside the block) layers of one cohort: rows [g B, (g + 1) B).
  // On return y holds the last FFN output and h the residual before it.
  auto plain_layers = [&](int g, int first, int last, bool defer_last) -> int {
    for (int i = first; i < last; ++i) {
      const int idx = i < ls ? i : ls + G * nl + (i - le);
      const Exec& ex = m->sched[idx];
      const loop_layer_weights& W = m->layers[i];
      if (int r = attention(i, g * B, B, {g}, {&ex}, true)) return r;
      LAUNCH(norm(g * B, B, true, W.ffn_norm), "add+rmsnorm");
      if (int r = ffn(i, g * B, B, defer_last || i + 1 < last)) return r;
      if (i + 1 < last) LAUNCH(norm(g * B, B, true, m->layers[i + 1].attn_norm), "add+rmsnorm");
    }
    return LOOP_OK;
  };

  // ---- the entering cohort: embedding and the layers before the block
  if (e >= 0) {
    LAUNCH(lk::embed(dt, tokens, m->embed, c.vocab, C, B, rows(h, e * B, C), (uint32_t*)st->base, s), "embed");
    if (ls > 0) {
      LAUNCH(norm(e * B, B, false, m->layers[0].attn_norm), "rmsnorm");
      if (int r = plain_layers(e, 0, ls, true)) return r;
    }
  }
  // ---- the block: every stored layer once, over all cohorts' rows
  std::vector<int> coh;
  for (int g = 0; g < G; ++g)
    if (pass[g]) coh.push_back(g);
  int mp = 1;     // maps[mp] holds the maps of the current site
  {
    const loop_layer_weights& W0 = m->layers[ls];
    if (e >= 0)   // streams enter: X = [h + y, h + y]
      LAUNCH(mhc(lk::MHC_ENTER, e * B, B, ls > 0 ? rows(y, e * B, C) : nullptr, ls > 0, nullptr, maps[1], W0.mhc_w[0],
                 W0.mhc_b[0], W0.attn_norm), "mhc enter");
    // every other cohort resumes from its park (cohorts with nothing in
    // flight go along as don't-care rows)
    for (int g = 0; g < G; ++g) {
      if (g == e) continue;
      int g1 = g;
      while (g1 + 1 < G && g1 + 1 != e) ++g1;
      LAUNCH(mhc(lk::MHC_MID, g * B, (g1 - g + 1) * B, rows(parkY, g * B, C), false, parkM, maps[1], W0.mhc_w[0],
                 W0.mhc_b[0], W0.attn_norm), "mhc resume");
      g = g1;
    }
  }
  for (int i = ls; i < le; ++i) {
    const loop_layer_weights& W = m->layers[i];
    std::vector<const Exec*> exs;
    for (int g : coh) exs.push_back(&m->sched[ls + (pass[g] - 1) * nl + (i - ls)]);
    if (int r = attention(i, 0, T, coh, exs, true)) return r;
    LAUNCH(mhc(lk::MHC_MID, 0, T, y, true, maps[mp], maps[mp ^ 1], W.mhc_w[1], W.mhc_b[1], W.ffn_norm), "mhc");
    mp ^= 1;
    const bool last = i + 1 == le;
    if (int r = ffn(i, 0, T, !last)) return r;
    if (!last) {
      const loop_layer_weights& Wn = m->layers[i + 1];
      LAUNCH(mhc(lk::MHC_MID, 0, T, y, true, maps[mp], maps[mp ^ 1], Wn.mhc_w[0], Wn.mhc_b[0], Wn.attn_norm), "mhc");
      mp ^= 1;
    }
  }
  // ---- leave the block: the cohort after pass P exits, the others park
  for (int g : coh) {
    if (g == f) continue;
    LAUNCH(hipMemcpyAsync(rows(parkY, g * B, C), rows(y, g * B, C), (size_t)B * C * es, hipMemcpyDeviceToDevice, s),
           "park y");
    LAUNCH(hipMemcpyAsync(parkM + (size_t)g * B * 8, maps[mp] + (size_t)g * B * 8, (size_t)B * 8 * sizeof(float),
                          hipMemcpyDeviceToDevice, s), "park maps");
  }
  if (f >= 0) {
    const float* gamma = le < c.n_layers ? m->layers[le].attn_norm : m->final_norm;
    LAUNCH(mhc(lk::MHC_EXIT, f * B, B, rows(y, f * B, C), false, maps[mp], nullptr, nullptr, nullptr, gamma),
           "mhc exit");
    if (le < c.n_layers) {
      if (int r = plain_layers(f, le, c.n_layers, true)) return r;
      LAUNCH(norm(f * B, B, true, m->final_norm), "add+rmsnorm");
    }
    LAUNCH(run_gemm(gemm(lk::EPI_F32, rows(u, f * B, C), C, B, m->head, c.vocab, C, logits, c.vocab), false),
           "head gemm");
  }
  // ---- bookkeeping
  for (int g : coh) {
    if (g == f) {
      st->pipe_next[g] = 0;
      for (int b = g * B; b < (g + 1) * B; ++b) st->seq_len[b] += 1;
    } else {
      st->pipe_next[g] = pass[g] + 1;
    }
  }
  if (e >= 0) st->pipe_enter = (e + 1) % G;
  info[0] = e;
  info[1] = f;
  return LOOP_OK;
}

}  // namespace

extern "C" {

int loop_prefill(loop_model* m, loop_state* st, void* workspace, size_t ws_bytes, const int32_t* tokens_dev,
                 const void* embeds_dev, int B, int S, unsigned flags, void* out_dev, void* stream) {
  if (!m) return lp_fail(LOOP_ERR_INVALID_ARG, "null model");
  if (flags & ~(unsigned)(LOOP_ALL_LOGITS | LOOP_HIDDEN_OUT | LOOP_CONTINUE))
    return lp_fail(LOOP_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  return forward(m, st, workspace, ws_bytes, 0, tokens_dev, embeds_dev, B, S, flags, out_dev, (hipStream_t)stream,
                 false);
}

int loop_prefill_rows(loop_model* m, loop_state* st, void* workspace, size_t ws_bytes, int seq0,
                      const int32_t* tokens_dev, const void* embeds_dev, int B, int S, unsigned flags, void* out_dev,
                      void* stream) {
  if (!m) return lp_fail(LOOP_ERR_INVALID_ARG, "null model");
  if (flags & ~(unsigned)(LOOP_ALL_LOGITS | LOOP_HIDDEN_OUT | LOOP_CONTINUE))
    return lp_fail(LOOP_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  return forward(m, st, workspace, ws_bytes, seq0, tokens_dev, embeds_dev, B, S, flags, out_dev, (hipStream_t)stream,
                 false);
}

int loop_decode_step(loop_model* m, loop_state* st, void* workspace, size_t ws_bytes, const int32_t* tokens_dev,
                     int B, float* logits_dev, void* stream) {
  if (!m) return lp_fail(LOOP_ERR_INVALID_ARG, "null model");
  if (!tokens_dev) return lp_fail(LOOP_ERR_INVALID_ARG, "null tokens");
  return forward(m, st, workspace, ws_bytes, 0, tokens_dev, nullptr, B, 1, 0, logits_dev, (hipStream_t)stream, true);
}

int loop_decode_step_noalloc(loop_model* m, loop_state* st, const int32_t* tokens_dev, int B, float* logits_dev,
                             void* stream) {
  if (!m) return lp_fail(LOOP_ERR_INVALID_ARG, "null model");
  if (!tokens_dev) return lp_fail(LOOP_ERR_INVALID_ARG, "null tokens");
  if (!st || st->m != m) return lp_fail(LOOP_ERR_STATE, "state does not belong to this model");
  if (B <= 0) return lp_fail(LOOP_ERR_INVALID_ARG, "B must be positive");
  const size_t need = ws_layout(m, B, B, st->max_seq).total;
  if (need > NOALLOC_WS_BYTES)
    return lp_fail(LOOP_ERR_WORKSPACE,
                   "a decode step of %d sequences (max_seq %d) needs %zu workspace bytes; the library's static "
                   "workspace holds %zu (use loop_decode_step with a caller workspace)",
                   B, st->max_seq, need, NOALLOC_WS_BYTES);
  void* ws = nullptr;
  if (int r = noalloc_scratch(&ws)) return r;
  return forward(m, st, ws, NOALLOC_WS_BYTES, 0, tokens_dev, nullptr, B, 1, 0, logits_dev, (hipStream_t)stream, true);
}

int loop_decode_pipelined(loop_model* m, loop_state* st, void* workspace, size_t ws_bytes, const int32_t* tokens_dev,
                          int B, float* logits_dev, int* cohorts, void* stream) {
  if (!m) return lp_fail(LOOP_ERR_INVALID_ARG, "null model");
  return decode_pipelined(m, st, workspace, ws_bytes, tokens_dev, B, logits_dev, cohorts, (hipStream_t)stream);
}

}  // extern "C"
