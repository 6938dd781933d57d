/*
 * loop_ops.h - op-level C ABI of libloop.so: each kernel family of the looped
 * decoder's forward pass on its own, on caller-owned device buffers.  The
 * model-level entry points (loop.h) are built from exactly these kernels; the
 * op-level ones exist to check each step against a reference at full size and
 * to time it.
 *
 * Conventions as in loop.h: row-major, 16-byte aligned device pointers,
 * asynchronous on `stream` (a hipStream_t as void*), LOOP_OK or a negative
 * loop_status (nothing is launched on error), deterministic results.
 * `dtype` is LOOP_FP32 or LOOP_BF16 for every non-float32 tensor.
 */
#ifndef LOOP_OPS_H
#define LOOP_OPS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { LOOP_EPI_STORE = 0, LOOP_EPI_F32 = 1, LOOP_EPI_SWIGLU = 3 };
enum { LOOP_MHC_ENTER = 0, LOOP_MHC_MID = 1, LOOP_MHC_EXIT = 2 };

/* Dense projection C = A . B^T, A [M][K] (row stride lda), B [N][K] (ldb),
 * fp32 accumulation (the QKV, O, gate/up, down and head projections).
 * epi STORE: C dtype [M][N]; F32: C float32 [M][N]; SWIGLU: B holds gate rows
 * [0, F) then up rows [F, 2F) (N = 2F) and C dtype [M][F] = silu(A.Bg^T) * (A.Bu^T).
 * bf16 with M > 64 needs K % 32 == 0, N (F for SWIGLU) a multiple of 256
 * (128 for SWIGLU) and 256 output rows within 2^31 bytes (ldc < 2^21 for
 * float32 output); bf16 with M <= 64 (the decode shape: the weights are
 * streamed once for up to 64 token rows) needs K % 64 == 0.
 * For M <= 64, `scratch` of loop_op_gemm_bytes() bytes (device, caller-owned,
 * contents arbitrary) lets K be split over workgroups when the output tiles
 * alone cannot fill the device; the partial sums are added in a fixed order,
 * so results are deterministic.  scratch NULL: no split (same kernel, one
 * workgroup per tile).  Errors: INVALID_ARG, SHAPE, ALIGN, WORKSPACE, HIP. */
size_t loop_op_gemm_bytes(int dtype, int epi, int M, int N, int K, int F);
int loop_op_gemm(int dtype, int epi, int M, int N, int K, const void* A, long lda, const void* B, long ldb,
                 void* C, long ldc, int F, void* scratch, size_t scratch_bytes, void* stream);

/* Residual add + RMSNorm outside the looped block: h <- h + y (y may be NULL),
 * u <- gamma * h / sqrt(mean(h^2) + eps).  h, y, u dtype [T][C]; gamma float32 [C]. */
int loop_op_add_rmsnorm(int dtype, int T, int C, const void* y, void* h, const float* gamma, void* u, float eps,
                        void* stream);

/* One two-stream hyper-connection transition per token (see loop.h for the
 * maps).  X dtype [T][2][C] in place; maps float32 [T][8] in the order
 * pre0 pre1 post0 post1 res00 res01 res10 res11.
 *  ENTER: X = [h + y, h + y] (y may be NULL); maps_out, u for site (w, b, gamma).
 *  MID:   X <- H_res X + H_post y with maps_in; then maps_out and u for (w, b, gamma).
 *  EXIT:  X' = H_res X + H_post y; h = (X'0 + X'1) / 2; u = RMSNorm(h; gamma).
 * C <= 4096, C % 8 == 0.  With bf16, C % 512 == 0 and T >= 256, ENTER and
 * MID run the projection W x on the matrix cores when `scratch` (>=
 * loop_op_mhc_bytes(C)) is given: W is split there into three bf16 parts
 * (high, middle, low; together within 2^-27 of W, so the projection equals a
 * float32 one up to summation order); otherwise (fewer tokens, or scratch
 * NULL) a float32 path with one workgroup per token runs. */
size_t loop_op_mhc_bytes(int C);
int loop_op_mhc(int dtype, int mode, int T, int C, int sinkhorn_iters, float eps, const void* y, void* h, void* X,
                const float* maps_in, float* maps_out, const float* w, const float* b, const float* gamma,
                void* u, void* scratch, size_t scratch_bytes, void* stream);

/* Causal softmax attention with grouped KV heads for S new positions (pos0 ..
 * pos0+S-1) of B sequences over a cache slot: K [B][Hkv][S_max][d],
 * V^T [B][Hkv][d][S_max] holding positions 0 .. pos0+S-1.  q: token (b, s) at
 * q + (b*S + s)*ldq, head j at + j*d; out likewise with ldo.  Query head j
 * reads KV head j / (Hq / Hkv); scale 1/sqrt(d).  bf16 needs d == 128 with
 * Hq / Hkv in {1, 2, 4, 8}, or d == 256 with Hq / Hkv in {1, 2, 4} (the 16
 * query / 4 KV heads of 256 in "How Does SenseNova-Loop Get More Depth Without
 * More Parameters?", section on the hybrid attention pattern), and
 * S_max % 64 == 0. */
int loop_op_attention(int dtype, int B, int S, int pos0, int S_max, int Hq, int Hkv, int d, const void* q, long ldq,
                      const void* kcache, const void* vcache, void* out, long ldo, void* stream);

/* The decode form: same contract (bf16: d 128 or 256), for Hq / Hkv * S <= 16.  The cache is split
 * over workgroups only as far as needed to fill the device (none at B * Hkv >=
 * the CU count); several splits are merged by a second kernel through
 * `scratch` (caller-owned, loop_op_attention_decode_bytes() bytes, an upper
 * bound for any Hkv and any pos0 + S <= S_max). */
size_t loop_op_attention_decode_bytes(int B, int S, int Hq, int d, int S_max);
int loop_op_attention_decode(int dtype, int B, int S, int pos0, int S_max, int Hq, int Hkv, int d, const void* q,
                             long ldq, const void* kcache, const void* vcache, void* out, long ldo, void* scratch,
                             size_t scratch_bytes, void* stream);
/* loop_op_attention_decode for a ragged batch: sequence b's S new queries sit
 * at positions pos_dev[b] .. pos_dev[b] + S - 1 (pos_dev: device int32 [B]).
 * max_pos0 bounds every start (0 <= pos_dev[b] <= max_pos0, max_pos0 + S <=
 * S_max): the split plan covers max_pos0 + S keys, and the kernels read each
 * start clamped to [0, max_pos0], so no access leaves the slots even for
 * starts outside that range (whose results are then not meaningful).  Same
 * scratch as loop_op_attention_decode.  dtype float32 runs the scalar kernel. */
int loop_op_attention_decode_ragged(int dtype, int B, int S, const int32_t* pos_dev, int max_pos0, int S_max, int Hq,
                                    int Hkv, int d, const void* q, long ldq, const void* kcache, const void* vcache,
                                    void* out, long ldo, void* scratch, size_t scratch_bytes, void* stream);

/* Decode attention for a ragged batch split stream-K (the split the model's
 * decode step uses when its sequences' lengths are far apart): the keys of
 * sequence b are positions 0 .. starts[b] + S - 1 (starts: host int32 [B]);
 * all sequences' keys, each padded to a multiple of 64, are laid end to end
 * and cut into pieces of one length per KV head, one workgroup per piece, and
 * a second kernel merges each (token, head) row's pieces.  bf16 only, d 128
 * or 256, (Hq / Hkv) * S <= 16, starts[b] + S <= S_max, S_max % 64 == 0.
 * `scratch` (caller-owned, loop_op_attention_decode_stream_k_bytes() bytes)
 * takes the partials and device copies of the starts and of the key prefix,
 * written on `stream` before the kernels run. */
size_t loop_op_attention_decode_stream_k_bytes(int B, int S, int Hq, int Hkv, int d);
int loop_op_attention_decode_stream_k(int dtype, int B, int S, const int32_t* starts, int S_max, int Hq, int Hkv,
                                      int d, const void* q, long ldq, const void* kcache, const void* vcache,
                                      void* out, long ldo, void* scratch, size_t scratch_bytes, void* stream);

/* Causal elu+1 linear attention for S new positions of B sequences from
 * qkv [B*S][ld] (q at column 0, k at Hq*d, v at (Hq+Hkv)*d), continuing the
 * float32 state S [B][Hkv][d][d], z [B][Hkv][d] (ignored and treated as zero
 * when init_zero), which is replaced by the state after the last position.
 * chunked = 1: chunk-parallel form (needs scratch of loop_op_linear_bytes());
 * chunked = 0: the recurrence, one position after another.  d: 64 or 128
 * (float32), 64, 128 or 256 (bf16). */
size_t loop_op_linear_bytes(int B, int S, int Hkv, int d);
int loop_op_linear(int dtype, int chunked, int B, int S, int Hq, int Hkv, int d, float eps, const void* qkv, long ld,
                   float* S_state, float* z_state, int init_zero, void* out, long ldo, void* scratch,
                   size_t scratch_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LOOP_OPS_H */
