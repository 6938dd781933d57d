// Causal linear attention with the elu+1 feature map and a normaliser, carried
// as a fixed-size per-(layer, pass) state S [B][Hkv][d][d], z [B][Hkv][d]
// (fp32):  S_t = S_{t-1} + phi(k_t) v_t^T, z_t = z_{t-1} + phi(k_t),
//          o_t = phi(q_t)^T S_t / (phi(q_t)^T z_t + eps).
//
// Prefill is chunk-parallel (chunks of 64 tokens):
//   lin_delta  : per chunk, dS_c = sum phi(k) v^T and dz_c     (all chunks at once)
//   lin_scan   : exclusive prefix over chunks, seeded by the incoming state;
//                the total becomes the outgoing state
//   lin_output : per chunk and query head,
//                o = (phi(Q) S_c + tril(phi(Q) phi(K)^T) V) / (phi(Q) z_c + rowsum + eps)
// Decode (a few tokens per sequence) runs the recurrence with S in registers.
#include "common.h"
#include "kernels.h"

namespace lk {

constexpr int LC = 64;   // chunk length

DEV float phi(float x) { return x > 0.f ? x + 1.0f : expf(x); }

size_t lin_scratch_floats(int B, int Hkv, int d, int S_call, int chunk) {
  const int nc = (S_call + chunk - 1) / chunk;
  return (size_t)B * Hkv * nc * ((size_t)d * d + d);
}

// ------------------------------------------------------------------ per-chunk deltas
template <typename T, int D>
__global__ __launch_bounds__(256) void lin_delta(LinArgs a) {
  extern __shared__ float lsm[];
  float* fk = lsm;              // [LC][D]
  float* vv = lsm + LC * D;     // [LC][D]
  constexpr int R = D / 16;
  const int c = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int nc = gridDim.x;
  const T* base = (const T*)a.qkv;
  for (int idx = threadIdx.x; idx < LC * D / 8; idx += 256) {
    const int t = idx / (D / 8), i8 = (idx % (D / 8)) * 8;
    const int s = c * LC + t;
    float kx[8], vx[8];
    if (s < a.S_call) {
      const T* row = base + (size_t)(b * a.S_call + s) * a.ld;
      ld8(row + (a.Hq + hk) * D + i8, kx);
      ld8(row + (a.Hq + a.Hkv + hk) * D + i8, vx);
#pragma unroll
      for (int e = 0; e < 8; ++e) kx[e] = phi(kx[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) { kx[e] = 0.f; vx[e] = 0.f; }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) { fk[t * D + i8 + e] = kx[e]; vv[t * D + i8 + e] = vx[e]; }
  }
  __syncthreads();
  const int ra = threadIdx.x / 16, cb = threadIdx.x % 16;
  float acc[R][R];
  float zacc[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    zacc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < R; ++j) acc[i][j] = 0.f;
  }
  for (int t = 0; t < LC; ++t) {
    float kr[R], vr[R];
#pragma unroll
    for (int i = 0; i < R; ++i) { kr[i] = fk[t * D + ra * R + i]; vr[i] = vv[t * D + cb * R + i]; }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      zacc[i] += kr[i];
#pragma unroll
      for (int j = 0; j < R; ++j) acc[i][j] += kr[i] * vr[j];
    }
  }
  float* out = a.scratch + ((size_t)bh * nc + c) * (D * D + D);
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int j = 0; j < R; ++j) out[(ra * R + i) * D + cb * R + j] = acc[i][j];
  if (cb == 0) {
#pragma unroll
    for (int i = 0; i < R; ++i) out[D * D + ra * R + i] = zacc[i];
  }
}

// ------------------------------------------------------------------ exclusive scan
__global__ __launch_bounds__(256) void lin_scan(LinArgs a, int nc) {
  const int D = a.d;
  const int E = D * D + D;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int bh = blockIdx.y;
  if (e >= E) return;
  float* st = (e < D * D) ? (a.S + (size_t)bh * D * D + e) : (a.z + (size_t)bh * D + (e - D * D));
  float run = a.init_zero ? 0.f : *st;
  float* p = a.scratch + (size_t)bh * nc * E + e;
  for (int c = 0; c < nc; ++c) {
    const float t = p[(size_t)c * E];
    p[(size_t)c * E] = run;
    run += t;
  }
  *st = run;
}

// ------------------------------------------------------------------ chunk outputs
template <typename T, int D>
__global__ __launch_bounds__(256) void lin_output(LinArgs a) {
  extern __shared__ float lsm[];
  float* fq = lsm;                       // [LC][D]
  float* R2 = fq + LC * D;               // fk [LC][D], later S_c [D][D] + z_c [D]
  float* Am = R2 + (D * D + D);          // [LC][LC]
  float* vv = Am + LC * LC;              // [LC][D]
  float* den = vv + LC * D;              // [LC]
  float* arow = den + LC;                // [LC]
  constexpr int R = D / 16;
  const int c = blockIdx.x, bj = blockIdx.y;
  const int b = bj / a.Hq, j = bj % a.Hq;
  const int G = a.Hq / a.Hkv, hk = j / G;
  const int nc = gridDim.x;
  const T* base = (const T*)a.qkv;

  for (int idx = threadIdx.x; idx < LC * D / 8; idx += 256) {
    const int t = idx / (D / 8), i8 = (idx % (D / 8)) * 8;
    const int s = c * LC + t;
    float qx[8], kx[8], vx[8];
    if (s < a.S_call) {
      const T* row = base + (size_t)(b * a.S_call + s) * a.ld;
      ld8(row + j * D + i8, qx);
      ld8(row + (a.Hq + hk) * D + i8, kx);
      ld8(row + (a.Hq + a.Hkv + hk) * D + i8, vx);
#pragma unroll
      for (int e = 0; e < 8; ++e) { qx[e] = phi(qx[e]); kx[e] = phi(kx[e]); }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) { qx[e] = 0.f; kx[e] = 0.f; vx[e] = 0.f; }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      fq[t * D + i8 + e] = qx[e];
      R2[t * D + i8 + e] = kx[e];
      vv[t * D + i8 + e] = vx[e];
    }
  }
  __syncthreads();
  {  // A = tril(phi(Q) phi(K)^T), 4x4 per thread
    const int ta = threadIdx.x / 16, tb = threadIdx.x % 16;
    float acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[x][y] = 0.f;
    for (int i = 0; i < D; ++i) {
      float qv[4], kv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) { qv[x] = fq[(ta * 4 + x) * D + i]; kv[x] = R2[(tb * 4 + x) * D + i]; }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] += qv[x] * kv[y];
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int t = ta * 4 + x, tau = tb * 4 + y;
        Am[t * LC + tau] = (tau <= t) ? acc[x][y] : 0.f;
      }
  }
  __syncthreads();
  {  // S_c, z_c replace phi(K)
    const float* src = a.scratch + ((size_t)(b * a.Hkv + hk) * nc + c) * (D * D + D);
    for (int idx = threadIdx.x; idx < (D * D + D) / 4; idx += 256)
      reinterpret_cast<float4*>(R2)[idx] = reinterpret_cast<const float4*>(src)[idx];
    if (threadIdx.x < LC) {
      float s = 0.f;
      for (int tau = 0; tau < LC; ++tau) s += Am[threadIdx.x * LC + tau];
      arow[threadIdx.x] = s;
    }
  }
  __syncthreads();
  if (threadIdx.x < LC) {
    const float* zc = R2 + D * D;
    float s = 0.f;
    for (int i = 0; i < D; ++i) s += fq[threadIdx.x * D + i] * zc[i];
    den[threadIdx.x] = s + arow[threadIdx.x] + a.eps;
  }
  __syncthreads();
  const int tr = threadIdx.x / 16, tc = threadIdx.x % 16;
  float num[4][R];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < R; ++y) num[x][y] = 0.f;
  for (int i = 0; i < D; ++i) {
    float qv[4], sv[R];
#pragma unroll
    for (int x = 0; x < 4; ++x) qv[x] = fq[(tr * 4 + x) * D + i];
#pragma unroll
    for (int y = 0; y < R; ++y) sv[y] = R2[i * D + tc * R + y];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < R; ++y) num[x][y] += qv[x] * sv[y];
  }
  for (int tau = 0; tau < LC; ++tau) {
    float av[4], vr[R];
#pragma unroll
    for (int x = 0; x < 4; ++x) av[x] = Am[(tr * 4 + x) * LC + tau];
#pragma unroll
    for (int y = 0; y < R; ++y) vr[y] = vv[tau * D + tc * R + y];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < R; ++y) num[x][y] += av[x] * vr[y];
  }
  T* out = (T*)a.out;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int t = tr * 4 + x;
    const int s = c * LC + t;
    if (s < a.S_call) {
      const float inv = 1.0f / den[t];
      T* o = out + (size_t)(b * a.S_call + s) * a.ldo + j * D + tc * R;
#pragma unroll
      for (int y = 0; y < R; ++y) st1(o + y, num[x][y] * inv);
    }
  }
}

// ------------------------------------------------------------------ chunk outputs, MFMA (d = 128)
// One workgroup per (chunk, sequence, KV head) serves the G query heads of the
// group, so S_c, z_c, phi(K) and V of the chunk are staged in LDS once.
// Products use v_mfma_f32_16x16x4f32 (float32 operands, the state stays
// float32).  Wave w owns chunk rows 16 w .. 16 w + 15.  In every product, lane
// group g = lane / 16 carries the contiguous slice g * K/4 .. of the
// contraction index on both operands (the sum is order-independent).
//   A_g   = tril(phi(Q_g) phi(K)^T)                 [64 x 64]
//   num_g = phi(Q_g) S_c + A_g V                      [64 x 128]
//   den_g = phi(Q_g) z_c + rowsum(A_g) + eps
typedef float f32x4v __attribute__((ext_vector_type(4)));
DEV f32x4v mfma_f32(float a, float b, f32x4v c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }

constexpr int LSP = 132;   // padded row of S^T and phi(K) (floats)
constexpr int LAP = 68;    // padded row of V^T and A (floats)
constexpr int LIN_MFMA_LDS = (128 * LSP + 64 * LSP + 128 * LAP + 64 * LAP + 128 + 64) * 4;

template <typename T>
__global__ __launch_bounds__(256, 1) void lin_output_mfma(LinArgs a) {
  extern __shared__ float lsm[];
  float* St = lsm;                  // [128][LSP]: St[j][k] = S_c[k][j]
  float* Kf = St + 128 * LSP;       // [64][LSP]: phi(K)[tau][d]
  float* Vt = Kf + 64 * LSP;        // [128][LAP]: Vt[j][tau] = V[tau][j]
  float* Am = Vt + 128 * LAP;       // [64][LAP]: masked A of the current head
  float* zc = Am + 64 * LAP;        // [128]
  float* den = zc + 128;            // [64]
  constexpr int D = 128;
  const int c = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int nc = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const T* base = (const T*)a.qkv;

  {  // stage S_c^T, z_c, phi(K), V^T
    const float* src = a.scratch + ((size_t)bh * nc + c) * (D * D + D);
    for (int idx = tid; idx < D * D / 4; idx += 256) {
      const int k = idx >> 5, j4 = (idx & 31) * 4;
      const float4 v = reinterpret_cast<const float4*>(src)[idx];
      St[(j4 + 0) * LSP + k] = v.x;
      St[(j4 + 1) * LSP + k] = v.y;
      St[(j4 + 2) * LSP + k] = v.z;
      St[(j4 + 3) * LSP + k] = v.w;
    }
    if (tid < D) zc[tid] = src[D * D + tid];
    for (int idx = tid; idx < LC * D / 8; idx += 256) {
      const int t = idx >> 4, i8 = (idx & 15) * 8;
      const int s = c * LC + t;
      float kx[8], vx[8];
      if (s < a.S_call) {
        const T* row = base + (size_t)(b * a.S_call + s) * a.ld;
        ld8(row + (a.Hq + hk) * D + i8, kx);
        ld8(row + (a.Hq + a.Hkv + hk) * D + i8, vx);
#pragma unroll
        for (int e = 0; e < 8; ++e) kx[e] = phi(kx[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { kx[e] = 0.f; vx[e] = 0.f; }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        Kf[t * LSP + i8 + e] = kx[e];
        Vt[(i8 + e) * LAP + t] = vx[e];
      }
    }
  }
  __syncthreads();

  const int t_row = 16 * w + li;                // A-operand row of this lane
  const int s_q = c * LC + t_row;
  for (int hq = 0; hq < G; ++hq) {
    const int j = hk * G + hq;
    // phi(q) of row t_row, d in [32 g, 32 g + 32)
    float q[32];
    if (s_q < a.S_call) {
      const T* row = base + (size_t)(b * a.S_call + s_q) * a.ld + j * D + 32 * g;
#pragma unroll
      for (int v8 = 0; v8 < 4; ++v8) {
        ld8(row + 8 * v8, q + 8 * v8);
#pragma unroll
        for (int e = 0; e < 8; ++e) q[8 * v8 + e] = phi(q[8 * v8 + e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) q[e] = 0.f;
    }
    // A blocks of this wave's rows: tau blocks nb <= w (later blocks are masked)
    for (int nb = 0; nb < 4; ++nb) {
      f32x4v acc = {0.f, 0.f, 0.f, 0.f};
      if (nb <= w) {
        const float* kr = Kf + (16 * nb + li) * LSP + 32 * g;
#pragma unroll
        for (int s4 = 0; s4 < 8; ++s4) {
          const float4 kv = *reinterpret_cast<const float4*>(kr + 4 * s4);
          acc = mfma_f32(q[4 * s4 + 0], kv.x, acc);
          acc = mfma_f32(q[4 * s4 + 1], kv.y, acc);
          acc = mfma_f32(q[4 * s4 + 2], kv.z, acc);
          acc = mfma_f32(q[4 * s4 + 3], kv.w, acc);
        }
      }
      // acc[r]: row 16 w + 4 g + r, column tau = 16 nb + li
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * w + 4 * g + r, tau = 16 * nb + li;
        Am[t * LAP + tau] = (tau <= t) ? acc[r] : 0.f;
      }
    }
    __syncthreads();
    {  // den for row t_row: phi(q) . z_c over the lane's slice + row sum of A over tau in [16 g, 16 g + 16)
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) p += q[e] * zc[32 * g + e];
#pragma unroll
      for (int e = 0; e < 16; ++e) p += Am[t_row * LAP + 16 * g + e];
      p += __shfl_xor(p, 16, 64);
      p += __shfl_xor(p, 32, 64);
      if (g == 0) den[t_row] = p + a.eps;
    }
    __syncthreads();
    float dinv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) dinv[r] = 1.0f / den[16 * w + 4 * g + r];
    T* out = (T*)a.out;
    for (int jb = 0; jb < 8; ++jb) {
      f32x4v acc = {0.f, 0.f, 0.f, 0.f};
      const float* sr = St + (16 * jb + li) * LSP + 32 * g;
#pragma unroll
      for (int s4 = 0; s4 < 8; ++s4) {
        const float4 sv = *reinterpret_cast<const float4*>(sr + 4 * s4);
        acc = mfma_f32(q[4 * s4 + 0], sv.x, acc);
        acc = mfma_f32(q[4 * s4 + 1], sv.y, acc);
        acc = mfma_f32(q[4 * s4 + 2], sv.z, acc);
        acc = mfma_f32(q[4 * s4 + 3], sv.w, acc);
      }
      const float* ar = Am + t_row * LAP + 16 * g;
      const float* vr = Vt + (16 * jb + li) * LAP + 16 * g;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const float4 av = *reinterpret_cast<const float4*>(ar + 4 * s4);
        const float4 vv4 = *reinterpret_cast<const float4*>(vr + 4 * s4);
        acc = mfma_f32(av.x, vv4.x, acc);
        acc = mfma_f32(av.y, vv4.y, acc);
        acc = mfma_f32(av.z, vv4.z, acc);
        acc = mfma_f32(av.w, vv4.w, acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * w + 4 * g + r;
        const int s = c * LC + t;
        if (s < a.S_call) st1(out + (size_t)(b * a.S_call + s) * a.ldo + j * D + 16 * jb + li, acc[r] * dinv[r]);
      }
    }
    __syncthreads();   // Am and den are rewritten by the next head
  }
}

// ------------------------------------------------------------------ decode (recurrent)
template <typename T, int D>
__global__ __launch_bounds__(256) void lin_decode_kernel(LinArgs a) {
  constexpr int NRG = 256 / D;          // row groups
  constexpr int RPT = D / NRG;          // rows per thread
  __shared__ float fk[D], vv[D], fq[8][D], zs[D], dens[8];
  __shared__ float red[NRG][8][D];
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int col = threadIdx.x % D, rg = threadIdx.x / D;
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* Sg = a.S + (size_t)bh * D * D;
  float s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) s[i] = a.init_zero ? 0.f : Sg[(rg * RPT + i) * D + col];
  float zr = 0.f;
  if (threadIdx.x < D) zr = a.init_zero ? 0.f : a.z[(size_t)bh * D + threadIdx.x];
  const T* base = (const T*)a.qkv;
  for (int t = 0; t < a.S_call; ++t) {
    const T* row = base + (size_t)(b * a.S_call + t) * a.ld;
    for (int idx = threadIdx.x; idx < (G + 2) * D; idx += 256) {
      const int part = idx / D, i = idx % D;
      if (part < G) fq[part][i] = phi(ld1(row + (hk * G + part) * D + i));
      else if (part == G) fk[i] = phi(ld1(row + (a.Hq + hk) * D + i));
      else vv[i] = ld1(row + (a.Hq + a.Hkv + hk) * D + i);
    }
    __syncthreads();
    const float vj = vv[col];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] += fk[rg * RPT + i] * vj;
    if (threadIdx.x < D) { zr += fk[threadIdx.x]; zs[threadIdx.x] = zr; }
    for (int g = 0; g < G; ++g) {
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) p += fq[g][rg * RPT + i] * s[i];
      red[rg][g][col] = p;
    }
    __syncthreads();
    for (int g = wid; g < G; g += 4) {
      float p = 0.f;
      for (int i = lane; i < D; i += 64) p += fq[g][i] * zs[i];
      p = wave_sum(p);
      if (lane == 0) dens[g] = p + a.eps;
    }
    __syncthreads();
    T* orow = (T*)a.out + (size_t)(b * a.S_call + t) * a.ldo;
    for (int idx = threadIdx.x; idx < G * D; idx += 256) {
      const int g = idx / D, jj = idx % D;
      float n = 0.f;
#pragma unroll
      for (int r = 0; r < NRG; ++r) n += red[r][g][jj];
      st1(orow + (hk * G + g) * D + jj, n / dens[g]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) Sg[(rg * RPT + i) * D + col] = s[i];
  if (threadIdx.x < D) a.z[(size_t)bh * D + threadIdx.x] = zr;
}

// ------------------------------------------------------------------ dispatch
template <typename T, int D>
static hipError_t prefill_t(const LinArgs& a, hipStream_t s) {
  const int nc = (a.S_call + LC - 1) / LC;
  const int BH = a.B * a.Hkv;
  const size_t lds1 = 2 * LC * D * sizeof(float);
  const size_t lds3 = (size_t)(LC * D + (D * D + D) + LC * LC + LC * D + 2 * LC) * sizeof(float);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)lin_delta<T, D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)lin_output<T, D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds3);
    if (e == hipSuccess && D == 128)
      e = hipFuncSetAttribute((const void*)lin_output_mfma<T>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              LIN_MFMA_LDS);
    if (e != hipSuccess) return e;
    attr = true;
  }
  lin_delta<T, D><<<dim3(nc, BH), 256, lds1, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int E = D * D + D;
  lin_scan<<<dim3((E + 255) / 256, BH), 256, 0, s>>>(a, nc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (D == 128) lin_output_mfma<T><<<dim3(nc, BH), 256, LIN_MFMA_LDS, s>>>(a);
  else lin_output<T, D><<<dim3(nc, a.B * a.Hq), 256, lds3, s>>>(a);
  return hipGetLastError();
}

hipError_t lin_prefill(const LinArgs& a, hipStream_t s) {
  if (a.S_call <= 0 || a.B <= 0) return hipSuccess;
  if (a.Hq % a.Hkv || a.Hq / a.Hkv > 8 || a.chunk != LC) return hipErrorInvalidValue;
  if (a.dt == DT_BF16) {
    if (a.d == 128) return prefill_t<bf16_t, 128>(a, s);
    if (a.d == 64) return prefill_t<bf16_t, 64>(a, s);
  } else {
    if (a.d == 128) return prefill_t<float, 128>(a, s);
    if (a.d == 64) return prefill_t<float, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t lin_decode(const LinArgs& a, hipStream_t s) {
  if (a.S_call <= 0 || a.B <= 0) return hipSuccess;
  if (a.Hq % a.Hkv || a.Hq / a.Hkv > 8) return hipErrorInvalidValue;
  const int grid = a.B * a.Hkv;
  if (a.dt == DT_BF16) {
    if (a.d == 128) lin_decode_kernel<bf16_t, 128><<<grid, 256, 0, s>>>(a);
    else if (a.d == 64) lin_decode_kernel<bf16_t, 64><<<grid, 256, 0, s>>>(a);
    else return hipErrorInvalidValue;
  } else {
    if (a.d == 128) lin_decode_kernel<float, 128><<<grid, 256, 0, s>>>(a);
    else if (a.d == 64) lin_decode_kernel<float, 64><<<grid, 256, 0, s>>>(a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lk
