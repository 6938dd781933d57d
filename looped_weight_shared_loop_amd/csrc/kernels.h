// Internal launch interface between the loop driver and the gfx950 kernels.
// Not part of the public C ABI (that is include/loop.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lk {

typedef uint16_t bf16_t;

enum Dt { DT_F32 = 0, DT_BF16 = 1 };

// ---------------------------------------------------------------- row kernels
hipError_t embed(int dt, const int32_t* tokens, const void* table, int vocab, int C, int T,
                 void* h, uint32_t* err_word, hipStream_t s);

// dst[0, n) <- vals[0, n) (host values passed as kernel arguments, so the
// host array may be reused as soon as the call returns).
hipError_t set_i32(int32_t* dst, const int32_t* vals, int n, hipStream_t s);

// h <- h + y (if y), u <- RMSNorm(h; gamma).  In place on h.
// A bf16 [T][C] sublayer output that is still split-K partial sums of the
// decode-shaped GEMM (tile of R output columns, ks partials of `tok` rows,
// tok = 32 or 64): element (t, c) =
// bf16(sum_p part[((c / R) * ks + p) * tok + t) * R + c % R]), the sum taken
// in index order as the GEMM's own reduction would.
struct YPart {
  const float* part;     // null: the output is stored in y
  int ks, rows, tok;
};

struct NormArgs {
  int dt, T, C;
  const void* y;
  YPart yp;              // overrides y when yp.part is set (bf16, T <= yp.tok)
  void* h;
  const float* gamma;
  void* u;
  float eps;
};
hipError_t add_rmsnorm(const NormArgs& a, hipStream_t s);

// Fused two-stream hyper-connection transition (write-back of one site, then
// maps, read and RMSNorm of the next site).
enum MhcMode { MHC_ENTER = 0, MHC_MID = 1, MHC_EXIT = 2 };
// rows of the bf16 split of an mHC projection W [8][2C]: high, middle and low parts
constexpr int MHC_WSPLIT_ROWS = 24;
constexpr int MHC_MFMA_MIN_T = 256;   // bf16 sites of at least this many tokens run tiled on MFMA

struct MhcArgs {
  int dt, mode, T, C, iters;
  float eps;
  const void* y;         // output of the sublayer just run (nullable on ENTER)
  YPart yp;              // overrides y when yp.part is set (bf16, per-token path only)
  void* h;               // ENTER: residual in; EXIT: residual out
  void* X;               // [T][2][C] streams, updated in place
  const float* maps_in;  // [T][8] maps of the site being written back (MID, EXIT)
  float* maps_out;       // [T][8] maps of the next site (ENTER, MID)
  const float* w;        // [8][2C] projection of the next site (ENTER, MID)
  const float* b;        // [8]
  const float* gamma;    // [C] RMSNorm gain of the next sublayer
  void* u;               // [T][C] normed input of the next sublayer
  int grid;              // persistent grid size (0: one block per token)
  bf16_t* wsplit;        // bf16 ENTER/MID: scratch of MHC_WSPLIT_ROWS x 2C bf16 for [W_hi; W_mid; W_lo]
  int wsplit_ready;      // the tiled path: wsplit already holds this W's split (no split launch)
};
hipError_t mhc(const MhcArgs& a, hipStream_t s);

// ---------------------------------------------------------------- GEMM
enum Epi { EPI_STORE = 0, EPI_F32 = 1, EPI_QKV = 2, EPI_SWIGLU = 3 };
// Paged KV cache of one full-attention slot: positions [64 j, 64 j + 64) of
// sequence b live in page table[b * stride + j] of the slot's page pool, K
// [n_pages][Hkv][64][d] and V^T [n_pages][Hkv][d][64] (every slot has its own
// pool; the table is shared).  Page numbers are clamped to [0, n_pages), so no
// table entry can make an access leave the pool.  table null: the contiguous
// layout K [B][Hkv][S_max][d], V^T [B][Hkv][d][S_max].
constexpr int KV_PAGE = 64;
struct KvPages {
  const int32_t* table;
  int stride, n_pages;
};
__device__ inline int kv_page(const KvPages& p, int b, int pos) {
  const int pg = p.table[(size_t)b * p.stride + (pos >> 6)];
  return min(max(pg, 0), p.n_pages - 1);
}
// element offset of K[b][hk][pos][0]
__device__ inline size_t kv_k_off(const KvPages& p, int Hkv, int S_max, int d, int b, int hk, int pos) {
  if (!p.table) return (((size_t)b * Hkv + hk) * S_max + pos) * d;
  return (((size_t)kv_page(p, b, pos) * Hkv + hk) * KV_PAGE + (pos & (KV_PAGE - 1))) * d;
}
// element offset of V^T[b][hk][0][pos]; rows of V^T are kv_vstride() apart
__device__ inline size_t kv_v_off(const KvPages& p, int Hkv, int S_max, int d, int b, int hk, int pos) {
  if (!p.table) return ((size_t)b * Hkv + hk) * d * S_max + pos;
  return ((size_t)kv_page(p, b, pos) * Hkv + hk) * d * KV_PAGE + (pos & (KV_PAGE - 1));
}
__host__ __device__ inline int kv_vstride(const KvPages& p, int S_max) { return p.table ? KV_PAGE : S_max; }

struct GemmArgs {
  int dt, epi;
  int M, N, K;          // C[M, N] = A[M, K] . B[N, K]^T; SWIGLU: N = 2F B rows, F outputs
  const void* A; long lda;
  const void* B; long ldb;
  void* C; long ldc;
  // EPI_QKV: columns [0, q_cols) -> C; [q_cols, q_cols + kv) -> K cache; then V cache
  int q_cols, n_kv, head_dim;
  void* kcache;          // [B][Hkv][S_max][d]
  void* vcache;          // [B][Hkv][d][S_max] (transposed)
  int S_call, pos0, S_max;  // row m is sequence m / S_call at position pos0 + m % S_call
  const int* pos_dev;    // non-null: sequence b starts at pos_dev[b] (ragged batch), read clamped
                         // to [0, pos0]: pos0 then holds the largest start, which bounds the writes
  KvPages pages;         // EPI_QKV, table non-null: kcache / vcache are page pools
  int F;                 // EPI_SWIGLU: up rows start at row F of B
  // M <= 64: split-K plan (skinny_plan) and its scratch; ksplit 1 needs none.
  int ksplit;
  int defer_reduce;      // ksplit > 1: leave the partials for the consumer (YPart)
  float* part;           // [tiles * ksplit][32 tb][128] fp32 partial sums, tb = M > 32 ? 2 : 1
};
hipError_t gemm(const GemmArgs& a, hipStream_t s);

// Decode-shaped (M <= 64) GEMM plan: 32 rb = 128 weight rows per workgroup
// tile (SwiGLU: 64 gate and 64 up rows) against tb = 1 or 2 blocks of 32 token
// rows, K split over `ksplit` workgroups when the tiles alone cannot fill the
// device.  `bytes` = partial sums (0 when ksplit == 1).
struct SkinnyPlan { int rb, tb, tiles, ksplit; size_t bytes; };
SkinnyPlan skinny_plan(int epi, int M, int N, int K, int F, int cu);

// ---------------------------------------------------------------- attention
struct AttnArgs {
  int dt, B, S_call, pos0, S_max, Hq, Hkv, d;
  const void* q; long ldq;         // token m: q + m * ldq, head j at + j * d
  const void* kcache;              // [B][Hkv][S_max][d]
  const void* vcache;              // [B][Hkv][d][S_max]
  void* out; long ldo;             // token m: out + m * ldo, head j at + j * d
  float* part; int n_split, split_len;   // decode: [B][Hq][n_split][d + 2] fp32 (n_split > 1)
  const int* pos_dev;              // decode: non-null: sequence b's new tokens start at pos_dev[b]
                                   // (ragged batch), read clamped to [0, pos0]: pos0 then holds
                                   // the largest start, which the split plan covers
  KvPages pages;                   // table non-null: kcache / vcache are page pools
};
hipError_t attn_prefill(const AttnArgs& a, hipStream_t s);
hipError_t attn_decode(const AttnArgs& a, hipStream_t s);
// K and V columns of B q|k|v rows (row stride ld, K from column q_cols) into a
// cache slot at position pos (one new position per sequence).
hipError_t kv_append(int dt, const void* qkv, long ld, int q_cols, int B, int Hkv, int d, void* kcache,
                     void* vcache, int S_max, int pos, KvPages pages, hipStream_t s);
// K and V of S rows per sequence (positions pos0 ..) from plainly stored
// q|k|v rows into a cache slot (paged or contiguous), V transposed.
hipError_t kv_scatter(int dt, const void* qkv, long ld, int q_cols, int B, int S, int pos0, const int* pos_dev,
                      int Hkv, int d, void* kcache, void* vcache, int S_max, KvPages pages, hipStream_t s);
// Decode split of the cache: as few splits as fill `cu` workgroups over the
// B * Hkv (sequence, KV head) pairs, each a multiple of 64 keys.
struct DecodePlan { int split_len, n_split; };
DecodePlan decode_plan(int B, int Hkv, int kv_len, int cu);
// Stream-K split of a ragged decode batch (attn_decode_sk): the sequences'
// keys, each padded to a multiple of 64, laid end to end (`total` keys) and
// cut into n_wg pieces of `chunk` keys per KV head; `slots` partials per row.
struct StreamKPlan { int chunk, n_wg, slots; };
int decode_sk_slots(int Hkv, int cu);
StreamKPlan decode_plan_sk(int total, int Hkv, int cu);
// pref: int32 [B + 1] device copy of the padded key prefix; a.pos_dev set.
hipError_t attn_decode_sk(const AttnArgs& a, const int32_t* pref, const StreamKPlan& p, hipStream_t s);
// upper bound of n_split over kv_len <= S_max
int decode_max_splits(int B, int Hkv, int S_max, int cu);

// ---------------------------------------------------------------- linear attention
struct LinArgs {
  int dt, B, S_call, Hq, Hkv, d;
  float eps;
  const void* qkv; long ld;        // q at column 0, k at Hq*d, v at (Hq+Hkv)*d
  float* S; float* z;              // [B][Hkv][d][d], [B][Hkv][d] fp32
  int init_zero;                   // treat the incoming state as zero
  void* out; long ldo;
  float* scratch; int chunk;       // prefill: [B*Hkv][n_chunk][d*d + d]
  YPart qp;                        // decode: qkv still split-K partials (bf16, S_call == 1)
};
hipError_t lin_prefill(const LinArgs& a, hipStream_t s);
hipError_t lin_decode(const LinArgs& a, hipStream_t s);
size_t lin_scratch_floats(int B, int Hkv, int d, int S_call, int chunk);

int device_cu_count();

}  // namespace lk
