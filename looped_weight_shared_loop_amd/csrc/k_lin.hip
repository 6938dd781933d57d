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
// bf16 with d = 128 or 256 runs the same three steps on the matrix cores (lin_delta_bf,
// lin_scan_t, lin_out_bf) with operands split into bf16 high and low parts.
// Decode (a few tokens per sequence) runs the recurrence with S in registers.
#include "common.h"
#include "kernels.h"

namespace lk {

constexpr int LC = 64;   // chunk length

DEV float phi(float x) { return x > 0.f ? x + 1.0f : expf(x); }
// the same with the hardware exponential (about 1 ulp), for the bf16 paths
DEV float phi_hw(float x) { return x > 0.f ? x + 1.0f : exp2_hw(x * 1.4426950408889634f); }

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

// ------------------------------------------------------------------ bf16, d = 128, matrix cores
// The same three steps on v_mfma_f32_32x32x16_bf16.  Every fp32 operand
// (phi(q), phi(k), the state, the intra-chunk weights A) is split into a bf16
// high part and the bf16 rounding of its remainder; a product takes
// hi.hi + hi.lo + lo.hi (lo.lo, about 2^-16 of the term, is dropped), with
// fp32 accumulation.  V is bf16 already and enters once.  Everything is
// computed transposed (rows = output feature j or key tau, columns = token):
// the chunk deltas and prefixes are stored as S^T [j][k].
constexpr int LP = LC + 8;      // LDS pitch (elements) of [128][64] tiles
constexpr int SP = 128 + 8;     // LDS pitch of [*][128] tiles

DEV void split_bf16(float x, bf16_t& hi, bf16_t& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}

// dS_c^T [j][k] = sum_tau V[tau][j] phi(K)[tau][k], dz_c = sum_tau phi(K)[tau].
// One workgroup per 128 x 128 block of dS_c^T: with head dim DK = 256 the
// grid's z index picks the value half jh and the key half kh.
template <int DK>
__global__ __launch_bounds__(256) void lin_delta_bf(LinArgs a) {
  constexpr int D = 128, KH = DK / 128;
  __shared__ __align__(16) bf16_t Kth[D * LP], Ktl[D * LP], Vt[D * LP];   // [feature][tau]
  __shared__ float zp[16][D];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int jh = blockIdx.z / KH, kh = blockIdx.z % KH;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int nc = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bf16_t* base = (const bf16_t*)a.qkv;
  {
    const int i8 = (tid & 15) * 8;          // this thread's 8 features
    float zs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    u32x4_t kraw[4], vraw[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int sq = min(c * LC + (tid >> 4) + 16 * s4, a.S_call - 1);
      const bf16_t* row = base + (size_t)(b * a.S_call + sq) * a.ld;
      kraw[s4] = ldv4(row + (a.Hq + hk) * DK + 128 * kh + i8);
      vraw[s4] = ldv4(row + (a.Hq + a.Hkv + hk) * DK + 128 * jh + i8);
    }
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int t = (tid >> 4) + 16 * s4;
      const bool ok = c * LC + t < a.S_call;
      float kx[8], vx[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wk = kraw[s4][e >> 1], wv = vraw[s4][e >> 1];
        kx[e] = ok ? phi(__uint_as_float((e & 1) ? (wk & 0xFFFF0000u) : (wk << 16))) : 0.f;
        vx[e] = ok ? __uint_as_float((e & 1) ? (wv & 0xFFFF0000u) : (wv << 16)) : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        zs[e] += kx[e];
        bf16_t hi, lo;
        split_bf16(kx[e], hi, lo);
        Kth[(i8 + e) * LP + t] = hi;
        Ktl[(i8 + e) * LP + t] = lo;
        Vt[(i8 + e) * LP + t] = f2bf(vx[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) zp[tid >> 4][i8 + e] = zs[e];
  }
  __syncthreads();
  // wave w: rows j in [32 w, 32 w + 32), all four 32-column blocks of k
  f32x16_t acc[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[kb][r] = 0.f;
  const int rl = lane & 31, h = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < LC / 16; ++ks) {
    const int tc = ks * 16 + h * 8;
    const bf16x8_t va = as_bf16x8(ldv4(Vt + (32 * w + rl) * LP + tc));
    bf16x8_t kh[4], kl[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      kh[kb] = as_bf16x8(ldv4(Kth + (32 * kb + rl) * LP + tc));
      kl[kb] = as_bf16x8(ldv4(Ktl + (32 * kb + rl) * LP + tc));
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) acc[kb] = mfma32(va, kh[kb], acc[kb]);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) acc[kb] = mfma32(va, kl[kb], acc[kb]);
  }
  float* out = a.scratch + ((size_t)bh * nc + c) * (DK * DK + DK);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = 32 * w + (r >> 2) * 8 + h * 4 + (r & 3);
      out[(128 * jh + j) * DK + 128 * kh + 32 * kb + rl] = acc[kb][r];
    }
  if (jh == 0 && tid < D) {
    float zt = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) zt += zp[g][tid];
    out[DK * DK + 128 * kh + tid] = zt;
  }
}

// Exclusive prefix over chunks of the transposed deltas, seeded by the
// incoming state S [k][j], z; the total becomes the outgoing state.
template <int D>
__global__ __launch_bounds__(256) void lin_scan_t(LinArgs a, int nc) {
  constexpr int E = D * D + D, U = 8;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int bh = blockIdx.y;
  if (e >= E) return;
  float* st = (e < D * D) ? (a.S + (size_t)bh * D * D + (e % D) * D + e / D) : (a.z + (size_t)bh * D + (e - D * D));
  float run = a.init_zero ? 0.f : *st;
  float* p = a.scratch + (size_t)bh * nc * E + e;
  int c = 0;
  for (; c + U <= nc; c += U) {
    float t[U];
#pragma unroll
    for (int u = 0; u < U; ++u) t[u] = p[(size_t)(c + u) * E];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      p[(size_t)(c + u) * E] = run;
      run += t[u];
    }
  }
  for (; c < nc; ++c) {
    const float t = p[(size_t)c * E];
    p[(size_t)c * E] = run;
    run += t;
  }
  *st = run;
}

// One workgroup per (chunk, sequence x KV head, up to four query heads of the
// group, value half), two waves per head (one per 32-token column block).
// Per head and value half jh (rows j of 128):
//   A^T  = mask(phi(K) phi(Q)^T)          [64 tau x 64 t]
//   num^T = S_c^T phi(Q)^T + V^T A^T      [128 j x 64 t]
//   den  = phi(Q) z_c + column sums of A^T + eps
// The key features (the contraction of A^T, of S_c^T phi(Q)^T and of den)
// come in KH = DK / 128 passes of 128, each staged into the same LDS.
constexpr int LIN_BF_LDS = (2 * 128 * SP + 2 * 64 * SP + 128 * LP) * 2 + 128 * 4;

template <int NH, int DK>
__global__ __launch_bounds__(128 * NH, 1) void lin_out_bf(LinArgs a) {
  constexpr int D = 128, KH = DK / 128;
  constexpr int nthr = 128 * NH;            // two waves per query head (NH heads here)
  extern __shared__ __align__(16) bf16_t lsb[];
  bf16_t* Sth = lsb;                  // [128 j][SP]: S_c^T high part (this pass's 128 key columns)
  bf16_t* Stl = Sth + 128 * SP;       // low part
  bf16_t* Kh = Stl + 128 * SP;        // [64 tau][SP]: phi(K) high
  bf16_t* Kl = Kh + 64 * SP;          // low
  bf16_t* Vt = Kl + 64 * SP;          // [128 j][LP]: V^T
  float* zc = (float*)(Vt + 128 * LP);
  const int c = blockIdx.x, bh = blockIdx.y;
  const int hg = blockIdx.z / KH, jh = blockIdx.z % KH;               // head group, value half
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int nc = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rl = lane & 31, h = lane >> 5;
  const bf16_t* base = (const bf16_t*)a.qkv;
  const int j_q = hk * (a.Hq / a.Hkv) + hg * NH + (w >> 1);          // this wave's query head
  const int tb = w & 1;                                               // and token block
  const int sq_mine = c * LC + tb * 32 + rl;                          // this lane's token
  const bool tok_ok = sq_mine < a.S_call;
  const float* src = a.scratch + ((size_t)bh * nc + c) * (DK * DK + DK);

  // num^T [128 j x 32 t] of this wave's token block and A^T blocks x <= tb
  f32x16_t num[4], at[2];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) num[db][r] = 0.f;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) at[x][r] = 0.f;
  float den = 0.f;

#pragma unroll 1
  for (int kh = 0; kh < KH; ++kh) {
    if (kh > 0) __syncthreads();            // every wave is done with the previous pass's LDS
    // this lane's q fragments for the pass's 8 k-steps, requested before the
    // staging so that they arrive while it runs
    u32x4_t qraw[8];
    {
      const bf16_t* qrow =
          base + (size_t)(b * a.S_call + min(sq_mine, a.S_call - 1)) * a.ld + j_q * DK + 128 * kh + h * 8;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qraw[ks] = ldv4(qrow + ks * 16);
    }
    {  // stage S_c^T (split), z_c, phi(K) (split, zero past the end) and, once, V^T
      constexpr int SPT = D * D / 4 / nthr;     // float4 per thread
      constexpr int SB = SPT < 16 ? SPT : 16;   // issued together
      constexpr int KPT = LC * D / 8 / nthr;    // 8-wide K / V items per thread
      constexpr int KB = KPT < 4 ? KPT : 4;
      if (tid < D) zc[tid] = src[DK * DK + 128 * kh + tid];
#pragma unroll
      for (int k0 = 0; k0 < KPT; k0 += KB) {
        u32x4_t kraw[KB], vraw[KB];
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          const int idx = tid + (k0 + i) * nthr;
          const int t = idx >> 4, i8 = (idx & 15) * 8;
          const int sq = min(c * LC + t, a.S_call - 1);
          const bf16_t* row = base + (size_t)(b * a.S_call + sq) * a.ld;
          kraw[i] = ldv4(row + (a.Hq + hk) * DK + 128 * kh + i8);
          if (kh == 0) vraw[i] = ldv4(row + (a.Hq + a.Hkv + hk) * DK + 128 * jh + i8);
        }
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          const int idx = tid + (k0 + i) * nthr;
          const int t = idx >> 4, i8 = (idx & 15) * 8;
          const bool ok = c * LC + t < a.S_call;
          bf16_t hi[8], lo[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t wk = kraw[i][e >> 1];
            const float kx = __uint_as_float((e & 1) ? (wk & 0xFFFF0000u) : (wk << 16));
            split_bf16(ok ? phi_hw(kx) : 0.f, hi[e], lo[e]);
            if (kh == 0) {
              const uint32_t wv = vraw[i][e >> 1];
              Vt[(i8 + e) * LP + t] = ok ? (bf16_t)((e & 1) ? (wv >> 16) : (wv & 0xFFFFu)) : (bf16_t)0;
            }
          }
          u32x4_t ph, pl;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ph[e] = hi[2 * e] | ((uint32_t)hi[2 * e + 1] << 16);
            pl[e] = lo[2 * e] | ((uint32_t)lo[2 * e + 1] << 16);
          }
          stv4(Kh + t * SP + i8, ph);
          stv4(Kl + t * SP + i8, pl);
        }
      }
#pragma unroll
      for (int s0 = 0; s0 < SPT; s0 += SB) {
        float4 sv[SB];
#pragma unroll
        for (int i = 0; i < SB; ++i) {
          const int idx = tid + (s0 + i) * nthr;
          const int j = idx >> 5, k4 = (idx & 31) * 4;
          sv[i] = *reinterpret_cast<const float4*>(src + (size_t)(128 * jh + j) * DK + 128 * kh + k4);
        }
#pragma unroll
        for (int i = 0; i < SB; ++i) {
          const int idx = tid + (s0 + i) * nthr;
          const int j = idx >> 5, k4 = (idx & 31) * 4;
          bf16_t hi[4], lo[4];
          split_bf16(sv[i].x, hi[0], lo[0]);
          split_bf16(sv[i].y, hi[1], lo[1]);
          split_bf16(sv[i].z, hi[2], lo[2]);
          split_bf16(sv[i].w, hi[3], lo[3]);
          *(u32x2_t*)(Sth + j * SP + k4) = u32x2_t{hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16)};
          *(u32x2_t*)(Stl + j * SP + k4) = u32x2_t{lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16)};
        }
      }
    }
    __syncthreads();

#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int dc = ks * 16 + h * 8;           // this lane's 8 features of the step
      float x8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wq = qraw[ks][e >> 1];
        x8[e] = tok_ok ? phi_hw(__uint_as_float((e & 1) ? (wq & 0xFFFF0000u) : (wq << 16))) : 0.f;
        den += x8[e] * zc[dc + e];
      }
      u32x4_t ph, pl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bf16_t h0, l0, h1, l1;
        split_bf16(x8[2 * e], h0, l0);
        split_bf16(x8[2 * e + 1], h1, l1);
        ph[e] = h0 | ((uint32_t)h1 << 16);
        pl[e] = l0 | ((uint32_t)l1 << 16);
      }
      const bf16x8_t qh = as_bf16x8(ph), ql = as_bf16x8(pl);
#pragma unroll
      for (int x = 0; x < 2; ++x)
        if (x <= tb) {
          const bf16x8_t kh8 = as_bf16x8(ldv4(Kh + (32 * x + rl) * SP + dc));
          const bf16x8_t kl8 = as_bf16x8(ldv4(Kl + (32 * x + rl) * SP + dc));
          at[x] = mfma32(kh8, qh, at[x]);
          at[x] = mfma32(kh8, ql, at[x]);
          at[x] = mfma32(kl8, qh, at[x]);
        }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8_t sh = as_bf16x8(ldv4(Sth + (32 * db + rl) * SP + dc));
        const bf16x8_t sl = as_bf16x8(ldv4(Stl + (32 * db + rl) * SP + dc));
        num[db] = mfma32(sh, qh, num[db]);
        num[db] = mfma32(sh, ql, num[db]);
        num[db] = mfma32(sl, qh, num[db]);
      }
      __builtin_amdgcn_sched_barrier(0);   // keep the steps apart: bounded register use
    }
  }
  // causal mask of the diagonal block: at[tb][r] holds tau = 32 tb + (r/4)*8 + 4h + r%4, t = 32 tb + rl
#pragma unroll
  for (int x = 0; x < 2; ++x)
    if (x == tb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if ((r >> 2) * 8 + h * 4 + (r & 3) > rl) at[x][r] = 0.f;
  // den: the two lane halves hold parts of phi(q) . z_c and of the column sums of A^T
#pragma unroll
  for (int x = 0; x < 2; ++x)
    if (x <= tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) den += at[x][r];
  den = x32_sum(den);
  // num^T += V^T A^T: k-step (x, half) covers tau 32x + 16half + {4h .. 4h+3, 8+4h .. 8+4h+3}
#pragma unroll
  for (int x = 0; x < 2; ++x)
    if (x <= tb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int t0 = 32 * x + 16 * half + 4 * h;
        bf16x8_t vf[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16_t* vr = Vt + (32 * db + rl) * LP;
          const u32x2_t lo8 = *(const u32x2_t*)(vr + t0);
          const u32x2_t hi8 = *(const u32x2_t*)(vr + t0 + 8);
          vf[db] = as_bf16x8(u32x4_t{lo8[0], lo8[1], hi8[0], hi8[1]});
        }
        u32x4_t ph, pl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf16_t h0, l0, h1, l1;
          split_bf16(at[x][half * 8 + 2 * e], h0, l0);
          split_bf16(at[x][half * 8 + 2 * e + 1], h1, l1);
          ph[e] = h0 | ((uint32_t)h1 << 16);
          pl[e] = l0 | ((uint32_t)l1 << 16);
        }
#pragma unroll
        for (int db = 0; db < 4; ++db) num[db] = mfma32(vf[db], as_bf16x8(ph), num[db]);
#pragma unroll
        for (int db = 0; db < 4; ++db) num[db] = mfma32(vf[db], as_bf16x8(pl), num[db]);
      }
  // out[t][j_q DK + 128 jh + j] = num^T[j][t] / den[t]; lane: column t, rows j in runs of 4
  if (tok_ok) {
    const float inv = 1.0f / (den + a.eps);
    bf16_t* orow = (bf16_t*)a.out + (size_t)(b * a.S_call + sq_mine) * a.ldo + j_q * DK + 128 * jh;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int j0 = 32 * db + g4 * 8 + h * 4;
        const uint32_t w0 = pack_bf16x2(num[db][g4 * 4] * inv, num[db][g4 * 4 + 1] * inv);
        const uint32_t w1 = pack_bf16x2(num[db][g4 * 4 + 2] * inv, num[db][g4 * 4 + 3] * inv);
        *(u32x2_t*)(orow + j0) = u32x2_t{w0, w1};
      }
  }
}

// ------------------------------------------------------------------ decode (recurrent)
// At decode shapes q, k and v may be read straight from the QKV projection's
// split-K partials.
template <typename T>
DEV float ld_qkv(const LinArgs& a, int row, int col) {
  if (a.qp.part) {
    const int R = a.qp.rows, tile = col / R;
    constexpr int KSMAX = 16;   // loads first, then the sum in index order
    float x[KSMAX];
#pragma unroll
    for (int p = 0; p < KSMAX; ++p)
      if (p < a.qp.ks) x[p] = a.qp.part[((size_t)(tile * a.qp.ks + p) * a.qp.tok + row) * R + (col - tile * R)];
    float v = 0.f;
#pragma unroll
    for (int p = 0; p < KSMAX; ++p)
      if (p < a.qp.ks) v += x[p];
    return round_to(v, (T*)nullptr);
  }
  return ld1((const T*)a.qkv + (size_t)row * a.ld + col);
}

// One workgroup per state, so that z is read and rewritten by one workgroup
// only.  Thread (row group rg, column jj) owns S[RPT rg .. RPT rg + RPT - 1]
// of a column; at d = 256 the columns come in four passes of 64 (the thread's
// rows of a pass are loaded, updated and stored each token), so that a thread
// never holds more than 64 state entries.
template <int D>
constexpr int lin_dec_cols() { return D == 256 ? 64 : D; }

template <typename T, int D>
__global__ __launch_bounds__(256) void lin_decode_kernel(LinArgs a) {
  constexpr int NJ = lin_dec_cols<D>();  // columns per pass
  constexpr int NP = D / NJ;             // passes over the columns
  constexpr int NRG = 256 / NJ;          // row groups (4, 2 or 4)
  constexpr int RPT = D / NRG;           // rows per thread (16, 64 or 64)
  __shared__ float fk[D], vv[D], fq[8][D], zs[D], dens[8];
  __shared__ float red[NRG][8][NJ];
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int jj = threadIdx.x % NJ, rg = threadIdx.x / NJ;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  float* Sg = a.S + (size_t)bh * D * D;
  float s[RPT];
  if (NP == 1) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = a.init_zero ? 0.f : Sg[(rg * RPT + i) * D + jj];
  }
  float zr = 0.f;
  if (threadIdx.x < D) zr = a.init_zero ? 0.f : a.z[(size_t)bh * D + threadIdx.x];
  for (int t = 0; t < a.S_call; ++t) {
    const int row = b * a.S_call + t;
    for (int idx = threadIdx.x; idx < (G + 2) * D; idx += 256) {
      const int part = idx / D, i = idx % D;
      if (part < G) fq[part][i] = phi(ld_qkv<T>(a, row, (hk * G + part) * D + i));
      else if (part == G) fk[i] = phi(ld_qkv<T>(a, row, (a.Hq + hk) * D + i));
      else vv[i] = ld_qkv<T>(a, row, (a.Hq + a.Hkv + hk) * D + i);
    }
    __syncthreads();
    if (threadIdx.x < D) { zr += fk[threadIdx.x]; zs[threadIdx.x] = zr; }
    T* orow = (T*)a.out + (size_t)row * a.ldo;
    for (int p = 0; p < NP; ++p) {
      const int col = p * NJ + jj;
      if (NP > 1) {   // this thread stored these entries itself at the previous token
#pragma unroll
        for (int i = 0; i < RPT; ++i) s[i] = (a.init_zero && t == 0) ? 0.f : Sg[(rg * RPT + i) * D + col];
      }
      const float vj = vv[col];
#pragma unroll
      for (int i = 0; i < RPT; ++i) s[i] += fk[rg * RPT + i] * vj;
      for (int g = 0; g < G; ++g) {
        float q = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) q += fq[g][rg * RPT + i] * s[i];
        red[rg][g][jj] = q;
      }
      if (NP > 1) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) Sg[(rg * RPT + i) * D + col] = s[i];
      }
      __syncthreads();
      if (p == 0) {
        for (int g = wid; g < G; g += 4) {
          float q = 0.f;
          for (int i = lane; i < D; i += 64) q += fq[g][i] * zs[i];
          q = wave_sum(q);
          if (lane == 0) dens[g] = q + a.eps;
        }
        __syncthreads();
      }
      for (int idx = threadIdx.x; idx < G * NJ; idx += 256) {
        const int g = idx / NJ, j = idx % NJ;
        float n = 0.f;
        for (int r = 0; r < NRG; ++r) n += red[r][g][j];
        st1(orow + (hk * G + g) * D + p * NJ + j, n / dens[g]);
      }
      __syncthreads();
    }
  }
  if (NP == 1) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) Sg[(rg * RPT + i) * D + jj] = s[i];
  }
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
  lin_output<T, D><<<dim3(nc, a.B * a.Hq), 256, lds3, s>>>(a);
  return hipGetLastError();
}

template <int NH, int DK>
static hipError_t launch_out_bf(const LinArgs& a, int nc, int BH, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    hipError_t e =
        hipFuncSetAttribute((const void*)lin_out_bf<NH, DK>, hipFuncAttributeMaxDynamicSharedMemorySize, LIN_BF_LDS);
    if (e != hipSuccess) return e;
    attr = true;
  }
  // groups of eight heads take two workgroups of four; d = 256 one more per value half
  lin_out_bf<NH, DK><<<dim3(nc, BH, a.Hq / a.Hkv / NH * (DK / 128)), 128 * NH, LIN_BF_LDS, s>>>(a);
  return hipGetLastError();
}

template <int DK>
static hipError_t prefill_bf(const LinArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return hipErrorInvalidValue;
  const int nc = (a.S_call + LC - 1) / LC;
  const int BH = a.B * a.Hkv;
  constexpr int KH = DK / 128;
  lin_delta_bf<DK><<<dim3(nc, BH, KH * KH), 256, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  lin_scan_t<DK><<<dim3((DK * DK + DK + 255) / 256, BH), 256, 0, s>>>(a, nc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // at d = 256 the state, the accumulators and the staging registers of
  // four heads do not fit two waves per SIMD: groups take workgroups of two heads
  switch (G) {
    case 1: return launch_out_bf<1, DK>(a, nc, BH, s);
    case 2: return launch_out_bf<2, DK>(a, nc, BH, s);
    default:
      if constexpr (DK == 128) return launch_out_bf<4, DK>(a, nc, BH, s);
      else return launch_out_bf<2, DK>(a, nc, BH, s);
  }
}

hipError_t lin_prefill(const LinArgs& a, hipStream_t s) {
  if (a.S_call <= 0 || a.B <= 0) return hipSuccess;
  if (a.Hq % a.Hkv || a.Hq / a.Hkv > 8 || a.chunk != LC) return hipErrorInvalidValue;
  if (a.dt == DT_BF16) {
    if (a.d == 128) return prefill_bf<128>(a, s);
    if (a.d == 256) return prefill_bf<256>(a, s);
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
  if (a.qp.part && (a.dt != DT_BF16 || a.S_call != 1 || a.qp.ks > 16)) return hipErrorInvalidValue;
  const int grid = a.B * a.Hkv;
  if (a.dt == DT_BF16) {
    if (a.d == 128) lin_decode_kernel<bf16_t, 128><<<grid, 256, 0, s>>>(a);
    else if (a.d == 256) lin_decode_kernel<bf16_t, 256><<<grid, 256, 0, s>>>(a);
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
