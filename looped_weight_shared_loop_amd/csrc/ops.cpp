// Op-level C ABI (include/loop_ops.h): one entry point per kernel family.
#include <hip/hip_runtime.h>

#include "../../include/loop.h"
#include "../../include/loop_ops.h"
#include "abi_util.h"
#include "kernels.h"
#include <vector>

namespace {

int dt_of(int dtype, int* dt) {
  if (dtype == LOOP_BF16) { *dt = lk::DT_BF16; return LOOP_OK; }
  if (dtype == LOOP_FP32) { *dt = lk::DT_F32; return LOOP_OK; }
  return lp_fail(LOOP_ERR_INVALID_ARG, "dtype %d", dtype);
}

int launched(hipError_t e, const char* what) {
  if (e == hipSuccess) return LOOP_OK;
  if (e == hipErrorInvalidValue) return lp_fail(LOOP_ERR_SHAPE, "%s: shape not supported by the kernel", what);
  return lp_fail(LOOP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool any_misaligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (lp_misaligned(p)) return true;
  return false;
}

constexpr int LIN_CHUNK = 64;

}  // namespace

extern "C" {

size_t loop_op_gemm_bytes(int dtype, int epi, int M, int N, int K, int F) {
  if (dtype != LOOP_BF16 || M <= 0 || M > 64 || N <= 0 || K <= 0) return 0;
  return lk::skinny_plan(epi, M, N, K, F, lk::device_cu_count()).bytes;
}

int loop_op_gemm(int dtype, int epi, int M, int N, int K, const void* A, long lda, const void* B, long ldb, void* C,
                 long ldc, int F, void* scratch, size_t scratch_bytes, void* stream) {
  int dt;
  if (int r = dt_of(dtype, &dt)) return r;
  if (!A || !B || !C) return lp_fail(LOOP_ERR_INVALID_ARG, "null pointer");
  if (epi != LOOP_EPI_STORE && epi != LOOP_EPI_F32 && epi != LOOP_EPI_SWIGLU)
    return lp_fail(LOOP_ERR_INVALID_ARG, "epilogue %d", epi);
  if (M < 0 || N <= 0 || K <= 0 || lda < K || ldb < K) return lp_fail(LOOP_ERR_INVALID_ARG, "sizes");
  if (epi == LOOP_EPI_SWIGLU && (F <= 0 || N != 2 * F || ldc < F)) return lp_fail(LOOP_ERR_INVALID_ARG, "swiglu sizes");
  if (epi != LOOP_EPI_SWIGLU && ldc < N) return lp_fail(LOOP_ERR_INVALID_ARG, "ldc");
  if (any_misaligned({A, B, C, scratch}) || lda % 8 || ldb % 8)
    return lp_fail(LOOP_ERR_ALIGN, "operands must be 16-byte aligned");
  lk::GemmArgs g{};
  g.dt = dt; g.epi = epi; g.M = M; g.N = N; g.K = K; g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc;
  g.F = F;
  g.ksplit = 1;
  if (dt == lk::DT_BF16 && M > 0 && M <= 64) {
    const lk::SkinnyPlan p = lk::skinny_plan(epi, M, N, K, F, lk::device_cu_count());
    if (p.ksplit > 1 && scratch) {
      if (scratch_bytes < p.bytes)
        return lp_fail(LOOP_ERR_WORKSPACE, "gemm scratch %zu bytes, needs %zu", scratch_bytes, p.bytes);
      g.ksplit = p.ksplit;
      g.part = (float*)scratch;
    }
  }
  return launched(lk::gemm(g, (hipStream_t)stream), "gemm");
}

int loop_op_add_rmsnorm(int dtype, int T, int C, const void* y, void* h, const float* gamma, void* u, float eps,
                        void* stream) {
  int dt;
  if (int r = dt_of(dtype, &dt)) return r;
  if (!h || !gamma || !u || T < 0 || C <= 0) return lp_fail(LOOP_ERR_INVALID_ARG, "arguments");
  if (any_misaligned({y, h, gamma, u})) return lp_fail(LOOP_ERR_ALIGN, "misaligned");
  lk::NormArgs a{};
  a.dt = dt; a.T = T; a.C = C; a.y = y; a.h = h; a.gamma = gamma; a.u = u; a.eps = eps;
  return launched(lk::add_rmsnorm(a, (hipStream_t)stream), "add_rmsnorm");
}

size_t loop_op_mhc_bytes(int C) { return C > 0 ? (size_t)lk::MHC_WSPLIT_ROWS * 2 * C * sizeof(uint16_t) : 0; }

int loop_op_mhc(int dtype, int mode, int T, int C, int iters, float eps, const void* y, void* h, void* X,
                const float* maps_in, float* maps_out, const float* w, const float* b, const float* gamma, void* u,
                void* scratch, size_t scratch_bytes, void* stream) {
  int dt;
  if (int r = dt_of(dtype, &dt)) return r;
  if (T < 0 || C <= 0 || iters < 0 || !X || !gamma || !u) return lp_fail(LOOP_ERR_INVALID_ARG, "arguments");
  if (mode == LOOP_MHC_ENTER) {
    if (!h || !maps_out || !w || !b) return lp_fail(LOOP_ERR_INVALID_ARG, "enter needs h, maps_out, w, b");
  } else if (mode == LOOP_MHC_MID) {
    if (!y || !maps_in || !maps_out || !w || !b) return lp_fail(LOOP_ERR_INVALID_ARG, "mid needs y, maps, w, b");
  } else if (mode == LOOP_MHC_EXIT) {
    if (!y || !maps_in || !h) return lp_fail(LOOP_ERR_INVALID_ARG, "exit needs y, maps_in, h");
  } else {
    return lp_fail(LOOP_ERR_INVALID_ARG, "mode %d", mode);
  }
  if (any_misaligned({y, h, X, w, gamma, u, scratch})) return lp_fail(LOOP_ERR_ALIGN, "misaligned");
  if (scratch && scratch_bytes < loop_op_mhc_bytes(C)) return lp_fail(LOOP_ERR_WORKSPACE, "mhc scratch too small");
  lk::MhcArgs a{};
  a.dt = dt; a.mode = mode; a.T = T; a.C = C; a.iters = iters; a.eps = eps; a.y = y; a.h = h; a.X = X;
  a.maps_in = maps_in; a.maps_out = maps_out; a.w = w; a.b = b; a.gamma = gamma; a.u = u;
  const int cu = lk::device_cu_count();
  a.grid = T < 2 * cu ? T : 2 * cu;
  a.wsplit = (lk::bf16_t*)scratch;
  return launched(lk::mhc(a, (hipStream_t)stream), "mhc");
}

static int attn_common(int dtype, int B, int S, int pos0, int S_max, int Hq, int Hkv, int d, const void* q, long ldq,
                       const void* k, const void* v, void* out, long ldo, lk::AttnArgs* a) {
  int dt;
  if (int r = dt_of(dtype, &dt)) return r;
  if (B <= 0 || S <= 0 || pos0 < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 || pos0 + S > S_max)
    return lp_fail(LOOP_ERR_INVALID_ARG, "sizes");
  if (!q || !k || !v || !out || ldq < Hq * d || ldo < Hq * d) return lp_fail(LOOP_ERR_INVALID_ARG, "pointers/strides");
  if (any_misaligned({q, k, v, out}) || ldq % 8 || ldo % 8) return lp_fail(LOOP_ERR_ALIGN, "misaligned");
  *a = lk::AttnArgs{};
  a->dt = dt; a->B = B; a->S_call = S; a->pos0 = pos0; a->S_max = S_max; a->Hq = Hq; a->Hkv = Hkv; a->d = d;
  a->q = q; a->ldq = ldq; a->kcache = k; a->vcache = v; a->out = out; a->ldo = ldo;
  return LOOP_OK;
}

int loop_op_attention(int dtype, int B, int S, int pos0, int S_max, int Hq, int Hkv, int d, const void* q, long ldq,
                      const void* kcache, const void* vcache, void* out, long ldo, void* stream) {
  lk::AttnArgs a;
  if (int r = attn_common(dtype, B, S, pos0, S_max, Hq, Hkv, d, q, ldq, kcache, vcache, out, ldo, &a)) return r;
  return launched(lk::attn_prefill(a, (hipStream_t)stream), "attention");
}

size_t loop_op_attention_decode_bytes(int B, int S, int Hq, int d, int S_max) {
  if (B <= 0 || S <= 0 || Hq <= 0 || d <= 0 || S_max <= 0) return 0;
  // bound over every KV-head count: the split count only falls as Hkv grows
  const size_t nsplit = (size_t)lk::decode_max_splits(B, 1, S_max, lk::device_cu_count());
  return (size_t)B * S * Hq * nsplit * (d + 2) * sizeof(float);
}

int loop_op_attention_decode(int dtype, int B, int S, int pos0, int S_max, int Hq, int Hkv, int d, const void* q,
                             long ldq, const void* kcache, const void* vcache, void* out, long ldo, void* scratch,
                             size_t scratch_bytes, void* stream) {
  lk::AttnArgs a;
  if (int r = attn_common(dtype, B, S, pos0, S_max, Hq, Hkv, d, q, ldq, kcache, vcache, out, ldo, &a)) return r;
  if (dtype == LOOP_FP32) return launched(lk::attn_prefill(a, (hipStream_t)stream), "attention");
  if (!scratch || scratch_bytes < loop_op_attention_decode_bytes(B, S, Hq, d, S_max))
    return lp_fail(LOOP_ERR_WORKSPACE, "decode attention scratch too small");
  if (lp_misaligned(scratch)) return lp_fail(LOOP_ERR_ALIGN, "misaligned scratch");
  const lk::DecodePlan dp = lk::decode_plan(B, Hkv, pos0 + S, lk::device_cu_count());
  a.part = (float*)scratch;
  a.split_len = dp.split_len;
  a.n_split = dp.n_split;
  return launched(lk::attn_decode(a, (hipStream_t)stream), "decode attention");
}

int loop_op_attention_decode_ragged(int dtype, int B, int S, const int32_t* pos_dev, int max_pos0, int S_max, int Hq,
                                    int Hkv, int d, const void* q, long ldq, const void* kcache, const void* vcache,
                                    void* out, long ldo, void* scratch, size_t scratch_bytes, void* stream) {
  if (!pos_dev) return lp_fail(LOOP_ERR_INVALID_ARG, "null positions");
  lk::AttnArgs a;
  if (int r = attn_common(dtype, B, S, max_pos0, S_max, Hq, Hkv, d, q, ldq, kcache, vcache, out, ldo, &a)) return r;
  a.pos_dev = pos_dev;
  if (dtype == LOOP_FP32) return launched(lk::attn_prefill(a, (hipStream_t)stream), "attention");
  if (!scratch || scratch_bytes < loop_op_attention_decode_bytes(B, S, Hq, d, S_max))
    return lp_fail(LOOP_ERR_WORKSPACE, "decode attention scratch too small");
  if (lp_misaligned(scratch)) return lp_fail(LOOP_ERR_ALIGN, "misaligned scratch");
  const lk::DecodePlan dp = lk::decode_plan(B, Hkv, max_pos0 + S, lk::device_cu_count());
  a.part = (float*)scratch;
  a.split_len = dp.split_len;
  a.n_split = dp.n_split;
  return launched(lk::attn_decode(a, (hipStream_t)stream), "decode attention");
}

size_t loop_op_attention_decode_stream_k_bytes(int B, int S, int Hq, int Hkv, int d) {
  if (B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return 0;
  const size_t slots = (size_t)lk::decode_sk_slots(Hkv, lk::device_cu_count());
  const size_t part = ((size_t)B * S * Hq * slots * (d + 2) * sizeof(float) + 255) / 256 * 256;
  return part + (size_t)(2 * B + 1) * sizeof(int32_t);
}

int loop_op_attention_decode_stream_k(int dtype, int B, int S, const int32_t* starts, int S_max, int Hq, int Hkv,
                                      int d, const void* q, long ldq, const void* kcache, const void* vcache,
                                      void* out, long ldo, void* scratch, size_t scratch_bytes, void* stream) {
  if (!starts) return lp_fail(LOOP_ERR_INVALID_ARG, "null starts");
  if (dtype != LOOP_BF16) return lp_fail(LOOP_ERR_INVALID_ARG, "the stream-K split runs bf16 only");
  int mx = 0;
  for (int b = 0; b < B; ++b) {
    if (starts[b] < 0) return lp_fail(LOOP_ERR_INVALID_ARG, "negative start");
    mx = starts[b] > mx ? starts[b] : mx;
  }
  lk::AttnArgs a;
  if (int r = attn_common(dtype, B, S, mx, S_max, Hq, Hkv, d, q, ldq, kcache, vcache, out, ldo, &a)) return r;
  if ((d != 128 && d != 256) || (Hq / Hkv) * S > 16 || S_max % 64)
    return lp_fail(LOOP_ERR_INVALID_ARG, "head size, group or S_max");
  const size_t need = loop_op_attention_decode_stream_k_bytes(B, S, Hq, Hkv, d);
  if (!scratch || scratch_bytes < need) return lp_fail(LOOP_ERR_WORKSPACE, "stream-K scratch too small");
  if (lp_misaligned(scratch)) return lp_fail(LOOP_ERR_ALIGN, "misaligned scratch");
  // scratch: partials, then the starts [B], then the padded key prefix [B + 1]
  int32_t* pos_dev = (int32_t*)((char*)scratch + need - (size_t)(2 * B + 1) * sizeof(int32_t));
  int32_t* pref_dev = pos_dev + B;
  std::vector<int32_t> pref(B + 1, 0);
  for (int b = 0; b < B; ++b) pref[b + 1] = pref[b] + (starts[b] + S + 63) / 64 * 64;
  const lk::StreamKPlan plan = lk::decode_plan_sk(pref[B], Hkv, lk::device_cu_count());
  hipStream_t s = (hipStream_t)stream;
  if (int r = launched(lk::set_i32(pos_dev, starts, B, s), "starts")) return r;
  if (int r = launched(lk::set_i32(pref_dev, pref.data(), B + 1, s), "key prefix")) return r;
  a.pos_dev = pos_dev;
  a.part = (float*)scratch;
  return launched(lk::attn_decode_sk(a, pref_dev, plan, s), "decode attention (stream-K)");
}

size_t loop_op_linear_bytes(int B, int S, int Hkv, int d) {
  if (B <= 0 || S <= 0 || Hkv <= 0 || d <= 0) return 0;
  return lk::lin_scratch_floats(B, Hkv, d, S, LIN_CHUNK) * sizeof(float);
}

int loop_op_linear(int dtype, int chunked, int B, int S, int Hq, int Hkv, int d, float eps, const void* qkv, long ld,
                   float* S_state, float* z_state, int init_zero, void* out, long ldo, void* scratch,
                   size_t scratch_bytes, void* stream) {
  int dt;
  if (int r = dt_of(dtype, &dt)) return r;
  if (B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 || !qkv || !S_state || !z_state || !out)
    return lp_fail(LOOP_ERR_INVALID_ARG, "arguments");
  if (ld < (long)(Hq + 2 * Hkv) * d || ldo < (long)Hq * d) return lp_fail(LOOP_ERR_INVALID_ARG, "strides");
  if (any_misaligned({qkv, S_state, z_state, out, scratch}) || ld % 8 || ldo % 8)
    return lp_fail(LOOP_ERR_ALIGN, "misaligned");
  lk::LinArgs a{};
  a.dt = dt; a.B = B; a.S_call = S; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.eps = eps; a.qkv = qkv; a.ld = ld;
  a.S = S_state; a.z = z_state; a.init_zero = init_zero; a.out = out; a.ldo = ldo;
  a.scratch = (float*)scratch; a.chunk = LIN_CHUNK;
  if (!chunked) return launched(lk::lin_decode(a, (hipStream_t)stream), "linear attention");
  if (!scratch || scratch_bytes < loop_op_linear_bytes(B, S, Hkv, d))
    return lp_fail(LOOP_ERR_WORKSPACE, "linear attention scratch too small");
  return launched(lk::lin_prefill(a, (hipStream_t)stream), "linear attention");
}

}  // extern "C"
