// Dense contractions of the looped decoder: C[M, N] = A[M, K] . B[N, K]^T.
//
// * gemm_mfma:   bf16, M > 32.  256x256x64 workgroup tile, 8 waves of
//                128x64 (4x2 blocks of v_mfma_f32_32x32x16_bf16), LDS double
//                buffer with an XOR swizzle of 16-byte chunks, XCD-aware tile
//                order.  fp32 accumulation.
// * gemm_skinny: bf16, M <= 32 (decode): streams B (the weights) once; each of
//                8 waves takes 1/8 of K for a 32-row block of B, then the
//                partial 32x32 blocks are summed in LDS in a fixed order.
// * gemm_f32:    fp32 configuration: LDS-tiled FMA kernel.
// All share one epilogue: plain bf16/fp32 store, fp32 logits, the QKV split
// that writes K and V into a per-(layer, pass) cache slot, or SwiGLU.
#include "common.h"
#include "kernels.h"

namespace lk {

// ------------------------------------------------------------------ epilogue
template <typename T>
DEV void epi_qkv(const GemmArgs& a, int row, int col, float v) {
  if (col < a.q_cols) {
    st1((T*)a.C + (size_t)row * a.ldc + col, v);
    return;
  }
  int cc = col - a.q_cols;
  const int kvn = a.n_kv * a.head_dim;
  const int b = row / a.S_call, pos = a.pos0 + row % a.S_call;
  if (cc < kvn) {
    const int hk = cc / a.head_dim, dd = cc % a.head_dim;
    st1((T*)a.kcache + (((size_t)b * a.n_kv + hk) * a.S_max + pos) * a.head_dim + dd, v);
  } else {
    cc -= kvn;
    const int hk = cc / a.head_dim, dd = cc % a.head_dim;
    st1((T*)a.vcache + (((size_t)b * a.n_kv + hk) * a.head_dim + dd) * a.S_max + pos, v);
  }
}

template <typename T, int EPI>
DEV void epi_one(const GemmArgs& a, int row, int col, float v) {
  if (EPI == EPI_STORE) st1((T*)a.C + (size_t)row * a.ldc + col, v);
  else if (EPI == EPI_F32) ((float*)a.C)[(size_t)row * a.ldc + col] = v;
  else if (EPI == EPI_QKV) epi_qkv<T>(a, row, col, v);
}

// ------------------------------------------------------------------ MFMA tile kernel
// 256x256x64 workgroup tile, 512 threads = 8 waves as 2 (M) x 4 (N); each
// wave owns a 128x64 sub-tile = 4x2 blocks of 32x32 (128 accumulators).
// SwiGLU: the B tile holds, per wave, 32 gate rows and the 32 matching up
// rows, so each wave emits 32 finished output columns (128 per workgroup).
constexpr int TBM = 256, TBN = 256, TBK = 64, GT = 512;
constexpr int GEMM_LDS = 2 * (TBM + TBN) * TBK * 2;   // 128 KB

DEV int swz(int row, int chunk) { return row * TBK + ((chunk ^ (row & 7)) << 3); }

template <int EPI>
__global__ __launch_bounds__(GT, 1) void gemm_mfma_kernel(GemmArgs a) {
  extern __shared__ __align__(16) bf16_t smem[];
  bf16_t* As = smem;                       // [2][TBM][TBK]
  bf16_t* Bs = smem + 2 * TBM * TBK;       // [2][TBN][TBK]

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 2, wn = wid & 3;
  const int num_m = (a.M + TBM - 1) / TBM;
  const int out_n = (EPI == EPI_SWIGLU) ? 128 : TBN;
  const int num_n = (EPI == EPI_SWIGLU ? a.F : a.N) / out_n;
  const int nblk = num_m * num_n;

  // XCD-aware order: consecutive hardware block ids go round-robin over the
  // 8 XCDs; give each XCD a contiguous range of tiles, then walk tiles in
  // groups of 8 row-tiles so neighbouring tiles share A and B panels in L2.
  int id = blockIdx.x;
  if (nblk % 8 == 0) id = (id & 7) * (nblk >> 3) + (id >> 3);
  const int GM = 8;
  const int group = GM * num_n;
  const int first_m = (id / group) * GM;
  const int gsz = min(num_m - first_m, GM);
  const int tm = first_m + (id % group) % gsz;
  const int tn = (id % group) / gsz;
  const int m0 = tm * TBM, n0 = tn * out_n;

  // Element offsets fit in 32 bits: the host checks M_tile*lda and N*ldb < 2^31.
  const bf16_t* A = (const bf16_t*)a.A + (long)m0 * a.lda;
  const bf16_t* B = (const bf16_t*)a.B;
  const int lrow = tid >> 3, lchunk = tid & 7;   // rows lrow + 64 i, i < 4
  const int mlast = a.M - 1 - m0;
  int aoff[4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = i * 64 + lrow;
    aoff[i] = min(r, mlast) * (int)a.lda + lchunk * 8;
    int br;
    if (EPI == EPI_SWIGLU) {
      const int w = r >> 6, j = (r >> 5) & 1, c = r & 31;
      br = (j == 0) ? (n0 + w * 32 + c) : (a.F + n0 + w * 32 + c);
    } else {
      br = n0 + r;
    }
    boff[i] = br * (int)a.ldb + lchunk * 8;
  }

  u32x4_t ra[4], rb[4];
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = a.K / TBK;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = ldv4(A + aoff[i]);
    rb[i] = ldv4(B + boff[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    stv4(As + swz(i * 64 + lrow, lchunk), ra[i]);
    stv4(Bs + swz(i * 64 + lrow, lchunk), rb[i]);
  }
  __syncthreads();

  const int arow = wm * 128 + (lane & 31);
  const int brow = wn * 64 + (lane & 31);
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) {
      const int k0 = (kt + 1) * TBK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = ldv4(A + aoff[i] + k0);
        rb[i] = ldv4(B + boff[i] + k0);
      }
    }
    const bf16_t* as = As + cur * TBM * TBK;
    const bf16_t* bs = Bs + cur * TBN * TBK;
#pragma unroll
    for (int ks = 0; ks < TBK / 16; ++ks) {
      const int ch = ks * 2 + (lane >> 5);
      bf16x8_t af[4], bfr[2];
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) af[ib] = as_bf16x8(ldv4(as + swz(arow + ib * 32, ch)));
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) bfr[jb] = as_bf16x8(ldv4(bs + swz(brow + jb * 32, ch)));
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) acc[ib][jb] = mfma32(af[ib], bfr[jb], acc[ib][jb]);
    }
    if (kt + 1 < KT) {
      bf16_t* an = As + (cur ^ 1) * TBM * TBK;
      bf16_t* bn = Bs + (cur ^ 1) * TBN * TBK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        stv4(an + swz(i * 64 + lrow, lchunk), ra[i]);
        stv4(bn + swz(i * 64 + lrow, lchunk), rb[i]);
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds column (lane & 31) and rows (r/4)*8 + (lane/32)*4 + r%4
  if (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + ib * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int col = n0 + wn * 32 + (lane & 31);
        if (row < a.M) {
          const float g = acc[ib][0][r], u = acc[ib][1][r];
          st1((bf16_t*)a.C + (size_t)row * a.ldc + col, silu(g) * u);
        }
      }
  } else {
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 128 + ib * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int col = n0 + wn * 64 + jb * 32 + (lane & 31);
          if (row < a.M) epi_one<bf16_t, EPI>(a, row, col, acc[ib][jb][r]);
        }
  }
}

// ------------------------------------------------------------------ skinny (M <= 32)
// Block of 32 B rows (SwiGLU: 16 gate + 16 matching up rows); 8 waves split K.
// MFMA A operand = B rows (weights), B operand = the <= 32 activation rows.
// Lane l: B row (l & 31), token (l & 31); its half h = l >> 5 owns a
// contiguous half of the wave's K range, 8 k per MFMA (the contraction index
// is permuted identically on both operands, which leaves the sum unchanged).
template <int EPI>
__global__ __launch_bounds__(512) void gemm_skinny_kernel(GemmArgs a) {
  __shared__ float red[8][32][33];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nb = blockIdx.x;
  const int r = lane & 31, h = lane >> 5;
  int brow;
  if (EPI == EPI_SWIGLU) brow = (r < 16) ? (nb * 16 + r) : (a.F + nb * 16 + (r - 16));
  else brow = nb * 32 + r;
  const int KW = a.K / 8;
  const int kbeg = wid * KW + h * (KW / 2);
  const int steps = KW / 16;
  const bf16_t* Bp = (const bf16_t*)a.B + (size_t)brow * a.ldb + kbeg;
  const bool tok_ok = r < a.M;
  const bf16_t* Ap = (const bf16_t*)a.A + (size_t)(tok_ok ? r : 0) * a.lda + kbeg;

  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  int s = 0;
  for (; s + 8 <= steps; s += 8) {
    u32x4_t wv[8], xv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      wv[j] = ldv4(Bp + (s + j) * 8);
      xv[j] = tok_ok ? ldv4(Ap + (s + j) * 8) : zero;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = mfma32(as_bf16x8(wv[j]), as_bf16x8(xv[j]), acc);
  }
  for (; s < steps; ++s) {
    const u32x4_t wv = ldv4(Bp + s * 8);
    const u32x4_t xv = tok_ok ? ldv4(Ap + s * 8) : zero;
    acc = mfma32(as_bf16x8(wv), as_bf16x8(xv), acc);
  }
  // acc: rows = B rows n = (i/4)*8 + h*4 + i%4, column = token (lane & 31)
#pragma unroll
  for (int i = 0; i < 16; ++i) red[wid][(i >> 2) * 8 + h * 4 + (i & 3)][lane & 31] = acc[i];
  __syncthreads();
  if (EPI == EPI_SWIGLU) {
    const int m = tid >> 4, c = tid & 15;
    if (m < a.M) {
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) { g += red[w][c][m]; u += red[w][16 + c][m]; }
      st1((bf16_t*)a.C + (size_t)m * a.ldc + nb * 16 + c, silu(g) * u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int idx = tid * 2 + e;
      const int m = idx >> 5, c = idx & 31;
      if (m < a.M) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) v += red[w][c][m];
        epi_one<bf16_t, EPI>(a, m, nb * 32 + c, v);
      }
    }
  }
}

// ------------------------------------------------------------------ fp32 kernel
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int BMf = 64, BNf = 64, BKf = 16;
  __shared__ float As[BKf][BMf + 4];
  __shared__ float Bs[BKf][BNf + 4];
  __shared__ float Us[BKf][BNf + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * BMf, n0 = blockIdx.x * BNf;
  const float* A = (const float*)a.A;
  const float* B = (const float*)a.B;
  float acc[4][4], accu[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) { acc[i][j] = 0.f; accu[i][j] = 0.f; }
  for (int k0 = 0; k0 < a.K; k0 += BKf) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + e * 256;           // 0..1023
      const int rr = idx >> 4, kk = idx & 15;  // rr 0..63
      const int gm = m0 + rr, gk = k0 + kk;
      As[kk][rr] = (gm < a.M && gk < a.K) ? A[(size_t)gm * a.lda + gk] : 0.f;
      const int gn = n0 + rr;
      const int nlim = (EPI == EPI_SWIGLU) ? a.F : a.N;
      Bs[kk][rr] = (gn < nlim && gk < a.K) ? B[(size_t)gn * a.ldb + gk] : 0.f;
      if (EPI == EPI_SWIGLU)
        Us[kk][rr] = (gn < nlim && gk < a.K) ? B[(size_t)(a.F + gn) * a.ldb + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKf; ++kk) {
      float av[4], bv[4], uv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bv[j] = Bs[kk][tx * 4 + j];
        if (EPI == EPI_SWIGLU) uv[j] = Us[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] += av[i] * bv[j];
          if (EPI == EPI_SWIGLU) accu[i][j] += av[i] * uv[j];
        }
    }
    __syncthreads();
  }
  const int nlim = (EPI == EPI_SWIGLU) ? a.F : a.N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + ty * 4 + i, col = n0 + tx * 4 + j;
      if (row < a.M && col < nlim) {
        if (EPI == EPI_SWIGLU)
          ((float*)a.C)[(size_t)row * a.ldc + col] = silu(acc[i][j]) * accu[i][j];
        else
          epi_one<float, EPI>(a, row, col, acc[i][j]);
      }
    }
}

// ------------------------------------------------------------------ dispatch
template <int EPI>
static hipError_t launch_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 32) {
    if (a.K % 128) return hipErrorInvalidValue;
    const int blocks = (EPI == EPI_SWIGLU) ? a.F / 16 : a.N / 32;
    if ((EPI == EPI_SWIGLU ? a.F % 16 : a.N % 32)) return hipErrorInvalidValue;
    gemm_skinny_kernel<EPI><<<blocks, 512, 0, s>>>(a);
    return hipGetLastError();
  }
  if (a.K % TBK) return hipErrorInvalidValue;
  if ((long)TBM * a.lda >= (1L << 31) || (long)(EPI == EPI_SWIGLU ? 2 * a.F : a.N) * a.ldb >= (1L << 31))
    return hipErrorInvalidValue;
  const int out_n = (EPI == EPI_SWIGLU) ? 128 : TBN;
  const int ncols = (EPI == EPI_SWIGLU) ? a.F : a.N;
  if (ncols % out_n) return hipErrorInvalidValue;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipSuccess;
    const void* fns[4] = {(const void*)gemm_mfma_kernel<EPI_STORE>, (const void*)gemm_mfma_kernel<EPI_F32>,
                          (const void*)gemm_mfma_kernel<EPI_QKV>, (const void*)gemm_mfma_kernel<EPI_SWIGLU>};
    for (int i = 0; i < 4 && e == hipSuccess; ++i)
      e = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, GEMM_LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int blocks = ((a.M + TBM - 1) / TBM) * (ncols / out_n);
  gemm_mfma_kernel<EPI><<<blocks, GT, GEMM_LDS, s>>>(a);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_f32(const GemmArgs& a, hipStream_t s) {
  const int ncols = (EPI == EPI_SWIGLU) ? a.F : a.N;
  dim3 grid((ncols + 63) / 64, (a.M + 63) / 64);
  gemm_f32_kernel<EPI><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t gemm(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.dt == DT_BF16) {
    switch (a.epi) {
      case EPI_STORE: return launch_bf16<EPI_STORE>(a, s);
      case EPI_F32: return launch_bf16<EPI_F32>(a, s);
      case EPI_QKV: return launch_bf16<EPI_QKV>(a, s);
      case EPI_SWIGLU: return launch_bf16<EPI_SWIGLU>(a, s);
    }
  } else {
    switch (a.epi) {
      case EPI_STORE: return launch_f32<EPI_STORE>(a, s);
      case EPI_F32: return launch_f32<EPI_F32>(a, s);
      case EPI_QKV: return launch_f32<EPI_QKV>(a, s);
      case EPI_SWIGLU: return launch_f32<EPI_SWIGLU>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace lk
