// Row kernels: embedding gather, residual add + RMSNorm outside the looped
// block, and the fused two-stream hyper-connection (mHC) transition inside it.
#include "common.h"
#include "kernels.h"

namespace lk {

// ------------------------------------------------------------------ embed
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tokens,
                                                    const T* __restrict__ table, int vocab, int C,
                                                    T* __restrict__ h, uint32_t* err) {
  const int r = blockIdx.x;
  int tok = tokens[r];
  if (tok < 0 || tok >= vocab) {
    if (threadIdx.x == 0) atomicOr(err, 1u);
    tok = 0;
  }
  const T* src = table + (size_t)tok * C;
  T* dst = h + (size_t)r * C;
  for (int i = threadIdx.x * 8; i < C; i += blockDim.x * 8) {
    float v[8];
    ld8(src + i, v);
    st8(dst + i, v);
  }
}

hipError_t embed(int dt, const int32_t* tokens, const void* table, int vocab, int C, int T,
                 void* h, uint32_t* err, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (dt == DT_BF16)
    embed_kernel<bf16_t><<<T, 256, 0, s>>>(tokens, (const bf16_t*)table, vocab, C, (bf16_t*)h, err);
  else
    embed_kernel<float><<<T, 256, 0, s>>>(tokens, (const float*)table, vocab, C, (float*)h, err);
  return hipGetLastError();
}

struct I32Block { int32_t v[64]; };

__global__ __launch_bounds__(64) void set_i32_kernel(int32_t* __restrict__ dst, I32Block b, int n) {
  if ((int)threadIdx.x < n) dst[threadIdx.x] = b.v[threadIdx.x];
}

hipError_t set_i32(int32_t* dst, const int32_t* vals, int n, hipStream_t s) {
  for (int i = 0; i < n; i += 64) {
    const int k = n - i < 64 ? n - i : 64;
    I32Block b{};
    for (int j = 0; j < k; ++j) b.v[j] = vals[i + j];
    set_i32_kernel<<<1, 64, 0, s>>>(dst + i, b, k);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ------------------------------------------------------------------ block sum
// Sums NV values over the block; `red` holds [2][16 waves][NV] floats and is
// used by token parity so one barrier per token suffices.
template <int NV>
DEV void block_sum(float* v, float (*red)[16][12], int par) {
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = wave_sum(v[i]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) red[par][wid][i] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = 0.f;
  for (int w = 0; w < nw; ++w) {
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] += red[par][w][i];
  }
}

// ------------------------------------------------------------------ add + RMSNorm
// 8 channels c0 .. c0 + 7 (one GEMM tile) of token t of a sublayer output:
// from y, or summed from the split-K partials and rounded like the stored y.
template <typename T, int PG = 4>
DEV void ld8_y(const T* y, const YPart& yp, int t, int C, int c0, float* v) {
  if (yp.part) {
    const int R = yp.rows, tile = c0 / R, j = c0 - tile * R;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
    // partial loads issued PG at a time ahead of their sums (index order kept)
    for (int p0 = 0; p0 < yp.ks; p0 += PG) {
      float4 lo[PG], hi[PG];
#pragma unroll
      for (int p = 0; p < PG; ++p)
        if (p0 + p < yp.ks) {
          const float4* q = reinterpret_cast<const float4*>(yp.part + ((size_t)(tile * yp.ks + p0 + p) * yp.tok + t) * R + j);
          lo[p] = q[0];
          hi[p] = q[1];
        }
#pragma unroll
      for (int p = 0; p < PG; ++p)
        if (p0 + p < yp.ks) {
          v[0] += lo[p].x; v[1] += lo[p].y; v[2] += lo[p].z; v[3] += lo[p].w;
          v[4] += hi[p].x; v[5] += hi[p].y; v[6] += hi[p].z; v[7] += hi[p].w;
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = round_to(v[e], (T*)nullptr);
    return;
  }
  ld8(y + (size_t)t * C + c0, v);
}

template <typename T, int MAXV>
__global__ __launch_bounds__(256) void add_rmsnorm_kernel(NormArgs a) {
  __shared__ float red[2][16][12];
  const int C = a.C, nv = C / 8;
  const T* y = (const T*)a.y;
  T* h = (T*)a.h;
  T* u = (T*)a.u;
  const int r = blockIdx.x;
  float x[MAXV][8];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < MAXV; ++k) {
    const int vi = threadIdx.x + k * blockDim.x;
    if (vi < nv) {
      ld8(h + (size_t)r * C + vi * 8, x[k]);
      if (y || a.yp.part) {
        float yv[8];
        ld8_y(y, a.yp, r, C, vi * 8, yv);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[k][e] = round_to(x[k][e] + yv[e], (T*)nullptr);
        st8(h + (size_t)r * C + vi * 8, x[k]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[k][e] * x[k][e];
    }
  }
  float tot[1] = {ss};
  block_sum<1>(tot, red, 0);
  const float inv = 1.0f / sqrtf(tot[0] / (float)C + a.eps);
#pragma unroll
  for (int k = 0; k < MAXV; ++k) {
    const int vi = threadIdx.x + k * blockDim.x;
    if (vi < nv) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = a.gamma[vi * 8 + e] * x[k][e] * inv;
      st8(u + (size_t)r * C + vi * 8, o);
    }
  }
}

hipError_t add_rmsnorm(const NormArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.C % 8 || a.C > 8192) return hipErrorInvalidValue;
  const int nv = a.C / 8;
  const int threads = nv >= 256 ? 256 : ((nv + 63) / 64) * 64;
  if (a.dt == DT_BF16)
    add_rmsnorm_kernel<bf16_t, 4><<<a.T, threads, 0, s>>>(a);
  else
    add_rmsnorm_kernel<float, 4><<<a.T, threads, 0, s>>>(a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ mHC
// One thread owns 8 consecutive channels c of both streams and keeps its
// slice of the next site's projection W (8 x 16 floats) in registers for the
// whole persistent loop over tokens, so W is read from memory once per block.
//
// Per token:  X'_i = sum_j H_res[i][j] X_j + H_post[i] y   (bf16-rounded, stored)
//             l = W vec(X') / rms(vec(X')) + b ; maps of the next site
//             u = gamma * x_in / rms(x_in), x_in = H_pre0 X'_0 + H_pre1 X'_1
// rms(x_in) comes from the three stream sums already reduced for l:
//   sum x_in^2 = p0^2 S00 + 2 p0 p1 S01 + p1^2 S11.
DEV void mhc_maps_from_logits(const float* l, int iters, float* m) {
  m[0] = 1.0f / (1.0f + expf(-l[0]));
  m[1] = 1.0f / (1.0f + expf(-l[1]));
  m[2] = 2.0f / (1.0f + expf(-l[2]));
  m[3] = 2.0f / (1.0f + expf(-l[3]));
  const float mx = fmaxf(fmaxf(l[4], l[5]), fmaxf(l[6], l[7]));
  float a = expf(l[4] - mx), b = expf(l[5] - mx), c = expf(l[6] - mx), d = expf(l[7] - mx);
  // rows, then columns, each scaled by the hardware reciprocal of its sum
  // (about 1 ulp; the iteration is a contraction, so these roundings do not
  // accumulate)
  for (int it = 0; it < iters; ++it) {
    const float i0 = __builtin_amdgcn_rcpf(a + b), i1 = __builtin_amdgcn_rcpf(c + d);
    a *= i0; b *= i0; c *= i1; d *= i1;
    const float j0 = __builtin_amdgcn_rcpf(a + c), j1 = __builtin_amdgcn_rcpf(b + d);
    a *= j0; c *= j0; b *= j1; d *= j1;
  }
  m[4] = a; m[5] = b; m[6] = c; m[7] = d;
}

template <typename T>
__global__ __launch_bounds__(512) void mhc_kernel(MhcArgs a) {
  __shared__ float red[2][16][12];
  const int C = a.C, nv = C / 8;
  const int v = threadIdx.x;
  const bool act = v < nv;
  const int c0 = act ? v * 8 : 0;
  T* X = (T*)a.X;
  T* h = (T*)a.h;
  T* u = (T*)a.u;
  const T* y = (const T*)a.y;
  const int mode = a.mode;

  float w[8][16];
  float bias[8];
  float g[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    bias[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) w[j][e] = 0.f;
  }
  if (mode != MHC_EXIT && act) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ld8(a.w + (size_t)j * 2 * C + c0, &w[j][0]);
      ld8(a.w + (size_t)j * 2 * C + C + c0, &w[j][8]);
      bias[j] = a.b[j];
    }
  }
  if (act) ld8(a.gamma + c0, g);

  int par = 0;
  for (int t = blockIdx.x; t < a.T; t += gridDim.x, par ^= 1) {
    float x0[8], x1[8];
    if (act) {
      if (mode == MHC_ENTER) {
        ld8(h + (size_t)t * C + c0, x0);
        if (y || a.yp.part) {
          float yv[8];
          ld8_y(y, a.yp, t, C, c0, yv);
#pragma unroll
          for (int e = 0; e < 8; ++e) x0[e] = round_to(x0[e] + yv[e], (T*)nullptr);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) x1[e] = x0[e];
        st8(X + ((size_t)t * 2) * C + c0, x0);
        st8(X + ((size_t)t * 2 + 1) * C + c0, x1);
      } else {
        float p[8], q[8], yv[8];
        ld8(X + ((size_t)t * 2) * C + c0, p);
        ld8(X + ((size_t)t * 2 + 1) * C + c0, q);
        ld8_y(y, a.yp, t, C, c0, yv);
        const float* mi = a.maps_in + (size_t)t * 8;
        const float po0 = mi[2], po1 = mi[3], r00 = mi[4], r01 = mi[5], r10 = mi[6], r11 = mi[7];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x0[e] = round_to(r00 * p[e] + r01 * q[e] + po0 * yv[e], (T*)nullptr);
          x1[e] = round_to(r10 * p[e] + r11 * q[e] + po1 * yv[e], (T*)nullptr);
        }
        if (mode == MHC_MID) {
          st8(X + ((size_t)t * 2) * C + c0, x0);
          st8(X + ((size_t)t * 2 + 1) * C + c0, x1);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) { x0[e] = 0.f; x1[e] = 0.f; }
    }

    if (mode == MHC_EXIT) {
      float hv[8];
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hv[e] = round_to(0.5f * (x0[e] + x1[e]), (T*)nullptr);
        ss += hv[e] * hv[e];
      }
      if (act) st8(h + (size_t)t * C + c0, hv);
      float tot[1] = {ss};
      block_sum<1>(tot, red, par);
      const float inv = 1.0f / sqrtf(tot[0] / (float)C + a.eps);
      if (act) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = g[e] * hv[e] * inv;
        st8(u + (size_t)t * C + c0, o);
      }
      continue;
    }

    float acc[11];
#pragma unroll
    for (int i = 0; i < 11; ++i) acc[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[0] += x0[e] * x0[e];
      acc[1] += x1[e] * x1[e];
      acc[2] += x0[e] * x1[e];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += w[j][e] * x0[e] + w[j][8 + e] * x1[e];
      acc[3 + j] = s;
    }
    block_sum<11>(acc, red, par);
    const float inv = 1.0f / sqrtf((acc[0] + acc[1]) / (float)(2 * C) + a.eps);
    float l[8], m[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) l[j] = acc[3 + j] * inv + bias[j];
    mhc_maps_from_logits(l, a.iters, m);
    if (threadIdx.x == 0) {
      float* mo = a.maps_out + (size_t)t * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) mo[j] = m[j];
    }
    const float p0 = m[0], p1 = m[1];
    const float ssin = p0 * p0 * acc[0] + 2.f * p0 * p1 * acc[2] + p1 * p1 * acc[1];
    const float invu = 1.0f / sqrtf(fmaxf(ssin, 0.f) / (float)C + a.eps);
    if (act) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = g[e] * (p0 * x0[e] + p1 * x1[e]) * invu;
      st8(u + (size_t)t * C + c0, o);
    }
  }
}

// ------------------------------------------------------------------ mHC, few tokens, channel split
// Decode-sized calls (T <= 64 tokens): one wave per (512-channel slice, token)
// instead of one workgroup per token, so a site fills the device.
//  A: the write-back (or the stream entry) of its slice, then the slice's
//     share of the 8 projections and of the three stream sums, stored to
//     part[t][slice][11];
//  B: the slices' shares summed in slice order, the maps (every wave of the
//     token computes them; slice 0 stores them), then u for its slice from
//     the X' that A wrote (the kernel boundary orders the two).
constexpr int MHC_SLICE = 512;

template <typename T>
__global__ __launch_bounds__(64) void mhc_slice_a(MhcArgs a, float* __restrict__ part) {
  const int C = a.C, nsl = C / MHC_SLICE;
  const int sl = blockIdx.x, t = blockIdx.y, lane = threadIdx.x;
  const int c0 = sl * MHC_SLICE + lane * 8;
  T* X = (T*)a.X;
  const T* y = (const T*)a.y;
  // the slice of W first: no load of the slice waits for another's result
  // or for the X' stores
  float w0[8][8], w1[8][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ld8(a.w + (size_t)j * 2 * C + c0, w0[j]);
    ld8(a.w + (size_t)j * 2 * C + C + c0, w1[j]);
  }
  float x0[8], x1[8];
  if (a.mode == MHC_ENTER) {
    ld8((const T*)a.h + (size_t)t * C + c0, x0);
    if (y || a.yp.part) {
      float yv[8];
      ld8_y<T, 16>(y, a.yp, t, C, c0, yv);
#pragma unroll
      for (int e = 0; e < 8; ++e) x0[e] = round_to(x0[e] + yv[e], (T*)nullptr);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x1[e] = x0[e];
  } else {
    float p[8], q[8], yv[8];
    ld8(X + ((size_t)t * 2) * C + c0, p);
    ld8(X + ((size_t)t * 2 + 1) * C + c0, q);
    ld8_y<T, 16>(y, a.yp, t, C, c0, yv);
    const float* mi = a.maps_in + (size_t)t * 8;
    const float po0 = mi[2], po1 = mi[3], r00 = mi[4], r01 = mi[5], r10 = mi[6], r11 = mi[7];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x0[e] = round_to(r00 * p[e] + r01 * q[e] + po0 * yv[e], (T*)nullptr);
      x1[e] = round_to(r10 * p[e] + r11 * q[e] + po1 * yv[e], (T*)nullptr);
    }
  }
  st8(X + ((size_t)t * 2) * C + c0, x0);
  st8(X + ((size_t)t * 2 + 1) * C + c0, x1);
  float acc[11];
  acc[0] = acc[1] = acc[2] = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc[0] += x0[e] * x0[e];
    acc[1] += x1[e] * x1[e];
    acc[2] += x0[e] * x1[e];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float sj = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sj += w0[j][e] * x0[e] + w1[j][e] * x1[e];
    acc[3 + j] = sj;
  }
#pragma unroll
  for (int i = 0; i < 11; ++i) acc[i] = wave_sum(acc[i]);
  if (lane < 11) {
    float v = acc[0];
#pragma unroll
    for (int i = 1; i < 11; ++i) v = lane == i ? acc[i] : v;
    part[((size_t)t * nsl + sl) * 11 + lane] = v;
  }
}

template <typename T>
__global__ __launch_bounds__(64) void mhc_slice_b(MhcArgs a, const float* __restrict__ part) {
  const int C = a.C, nsl = C / MHC_SLICE;
  const int sl = blockIdx.x, t = blockIdx.y, lane = threadIdx.x;
  const int c0 = sl * MHC_SLICE + lane * 8;
  // the slice's X' and gain do not depend on the maps: in flight during them
  float x0[8], x1[8], g[8], o[8];
  ld8((const T*)a.X + ((size_t)t * 2) * C + c0, x0);
  ld8((const T*)a.X + ((size_t)t * 2 + 1) * C + c0, x1);
  ld8(a.gamma + c0, g);
  float acc[11];
#pragma unroll
  for (int i = 0; i < 11; ++i) acc[i] = 0.f;
  for (int q = 0; q < nsl; ++q) {
    const float* pq = part + ((size_t)t * nsl + q) * 11;
#pragma unroll
    for (int i = 0; i < 11; ++i) acc[i] += pq[i];
  }
  const float inv = 1.0f / sqrtf((acc[0] + acc[1]) / (float)(2 * C) + a.eps);
  float l[8], m[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) l[j] = acc[3 + j] * inv + a.b[j];
  mhc_maps_from_logits(l, a.iters, m);
  if (sl == 0 && lane == 0) {
    float* mo = a.maps_out + (size_t)t * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) mo[j] = m[j];
  }
  const float p0 = m[0], p1 = m[1];
  const float ssin = p0 * p0 * acc[0] + 2.f * p0 * p1 * acc[2] + p1 * p1 * acc[1];
  const float invu = 1.0f / sqrtf(fmaxf(ssin, 0.f) / (float)C + a.eps);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = g[e] * (p0 * x0[e] + p1 * x1[e]) * invu;
  st8((T*)a.u + (size_t)t * C + c0, o);
}

// ------------------------------------------------------------------ mHC, MFMA (bf16)
// For bf16 streams the 8 projections l = W vec(X') run on the matrix cores:
// W (float32 [8][2C]) is split (once per call, or kept by the caller across
// calls with the same W: wsplit_ready) into W_hi = bf16(W),
// W_mid = bf16(W - W_hi) and W_lo = bf16(W - W_hi - W_mid), 24 bf16 rows
// that carry W to within 2^-27 of its value (finer than float32's own
// rounding): X' is bf16, so each product is exact and the projection equals
// a float32 one up to the order of the float32 sums.  One
// v_mfma_f32_16x16x32_bf16 takes [W_hi; W_mid] (columns j and j + 8), a
// second one W_lo (columns j < 8); l_j = col j + col j+8 over both.
// A workgroup of 8 waves handles 16 tokens at a time; wave w owns channels
// [w C/8, (w+1) C/8) of both streams, lane l owns token l % 16 and 8 channels
// per 32-channel step.  The Sinkhorn maps are computed once per token (one
// lane each), then every lane forms u from the X' it wrote.
__global__ __launch_bounds__(256) void mhc_split_w(const float* __restrict__ w, bf16_t* __restrict__ ws, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const float v = w[i];
    const bf16_t hi = f2bf(v);
    const float r1 = v - bf2f(hi);    // exact in float32
    const bf16_t mid = f2bf(r1);
    ws[i] = hi;                       // rows 0..7
    ws[n + i] = mid;                  // rows 8..15
    ws[2 * n + i] = f2bf(r1 - bf2f(mid));   // rows 16..23
  }
}

__global__ __launch_bounds__(512) void mhc_mfma_kernel(MhcArgs a, const bf16_t* __restrict__ wsplit) {
  constexpr int NSMAX = 16;                 // C <= 4096: 32-channel steps per wave
  constexpr int GRP = 2;                    // steps whose loads are issued together
  __shared__ float red_acc[8][16][17];
  __shared__ float red_s[8][16][3];
  __shared__ float tl[16][17];
  __shared__ float ts[16][3];
  __shared__ float mp[16][3];
  const int C = a.C, C2 = 2 * C;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int CW = C / 8, NS = CW / 32;
  const int mode = a.mode;
  bf16_t* X = (bf16_t*)a.X;
  const bf16_t* hin = (const bf16_t*)a.h;
  const bf16_t* y = (const bf16_t*)a.y;
  bf16_t* u = (bf16_t*)a.u;
  const int ntiles = (a.T + 15) / 16;
  const bf16_t* wrow = wsplit + (size_t)li * C2;   // row li of [W_hi; W_mid]
  const bool has_lo = li < 8;
  const bf16_t* wlo = wsplit + (size_t)(16 + (has_lo ? li : 0)) * C2;   // row li of W_lo
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int t = tile * 16 + li;
    const bool tv = t < a.T;
    float po0 = 0.f, po1 = 0.f, r00 = 0.f, r01 = 0.f, r10 = 0.f, r11 = 0.f;
    if (mode == MHC_MID && tv) {
      const float* mi = a.maps_in + (size_t)t * 8;
      po0 = mi[2]; po1 = mi[3]; r00 = mi[4]; r01 = mi[5]; r10 = mi[6]; r11 = mi[7];
    }
    const size_t tr = tv ? (size_t)t : 0;
    const bf16_t* X0r = X + (tr * 2) * C + w * CW + 8 * g;
    const bf16_t* X1r = X0r + C;
    const bf16_t* Hr = hin + tr * C + w * CW + 8 * g;
    const bf16_t* Yr = (y ? y + tr * C : nullptr) + w * CW + 8 * g;
    // X' of this lane's token and channels stays in registers (bf16 pairs)
    u32x4_t xs0[NSMAX], xs1[NSMAX];
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, acc_lo = {0.f, 0.f, 0.f, 0.f};
    float s00 = 0.f, s11 = 0.f, s01 = 0.f;
#pragma unroll
    for (int j0 = 0; j0 < NSMAX; j0 += GRP) {
      if (j0 < NS) {
        u32x4_t la[GRP], lb[GRP], lc[GRP];
#pragma unroll
        for (int k = 0; k < GRP; ++k) {
          const int off = 32 * (j0 + k);
          if (mode == MHC_ENTER) {
            la[k] = tv ? ldv4(Hr + off) : zero;
            lc[k] = (tv && y) ? ldv4(Yr + off) : zero;
          } else {
            la[k] = tv ? ldv4(X0r + off) : zero;
            lb[k] = tv ? ldv4(X1r + off) : zero;
            lc[k] = tv ? ldv4(Yr + off) : zero;
          }
        }
#pragma unroll
        for (int k = 0; k < GRP; ++k) {
          const int j = j0 + k;
          float x0[8], x1[8];
          if (mode == MHC_ENTER) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t wa = la[k][e >> 1], wc = lc[k][e >> 1];
              const float hv = __uint_as_float((e & 1) ? (wa & 0xFFFF0000u) : (wa << 16));
              const float yv = __uint_as_float((e & 1) ? (wc & 0xFFFF0000u) : (wc << 16));
              x0[e] = bf2f(f2bf(hv + yv));   // y absent: adds 0
              x1[e] = x0[e];
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t wa = la[k][e >> 1], wb = lb[k][e >> 1], wc = lc[k][e >> 1];
              const float p = __uint_as_float((e & 1) ? (wa & 0xFFFF0000u) : (wa << 16));
              const float q = __uint_as_float((e & 1) ? (wb & 0xFFFF0000u) : (wb << 16));
              const float yv = __uint_as_float((e & 1) ? (wc & 0xFFFF0000u) : (wc << 16));
              x0[e] = bf2f(f2bf(r00 * p + r01 * q + po0 * yv));
              x1[e] = bf2f(f2bf(r10 * p + r11 * q + po1 * yv));
            }
          }
          u32x4_t p0, p1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // exact: the values are already bf16
            p0[e] = (__float_as_uint(x0[2 * e]) >> 16) | (__float_as_uint(x0[2 * e + 1]) & 0xFFFF0000u);
            p1[e] = (__float_as_uint(x1[2 * e]) >> 16) | (__float_as_uint(x1[2 * e + 1]) & 0xFFFF0000u);
          }
          xs0[j] = p0;
          xs1[j] = p1;
          if (tv) {
            stv4(X + (tr * 2) * C + w * CW + 32 * j + 8 * g, p0);
            stv4(X + (tr * 2 + 1) * C + w * CW + 32 * j + 8 * g, p1);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            s00 += x0[e] * x0[e];
            s11 += x1[e] * x1[e];
            s01 += x0[e] * x1[e];
          }
          const int cb = w * CW + 32 * j + 8 * g;
          const bf16x8_t w0 = as_bf16x8(ldv4(wrow + cb));
          const bf16x8_t w1 = as_bf16x8(ldv4(wrow + C + cb));
          acc = mfma16(as_bf16x8(p0), w0, acc);
          acc = mfma16(as_bf16x8(p1), w1, acc);
          const bf16x8_t v0 = as_bf16x8(has_lo ? ldv4(wlo + cb) : zero);
          const bf16x8_t v1 = as_bf16x8(has_lo ? ldv4(wlo + C + cb) : zero);
          acc_lo = mfma16(as_bf16x8(p0), v0, acc_lo);
          acc_lo = mfma16(as_bf16x8(p1), v1, acc_lo);
        }
      }
    }
    // acc[r]: token 4 g + r, column li; the stream sums of token li are split over the 4 groups
    // columns j < 8: hi + lo parts of logit j; columns j + 8: its mid part
#pragma unroll
    for (int r = 0; r < 4; ++r) red_acc[w][4 * g + r][li] = acc[r] + acc_lo[r];
    s00 = x32_sum(x16_sum(s00));
    s11 = x32_sum(x16_sum(s11));
    s01 = x32_sum(x16_sum(s01));
    if (g == 0) { red_s[w][li][0] = s00; red_s[w][li][1] = s11; red_s[w][li][2] = s01; }
    __syncthreads();
    if (tid < 256) {
      const int ti = tid >> 4, cc = tid & 15;
      float v = 0.f;
#pragma unroll
      for (int ww = 0; ww < 8; ++ww) v += red_acc[ww][ti][cc];
      tl[ti][cc] = v;
    } else if (tid < 256 + 48) {
      const int ti = (tid - 256) / 3, k = (tid - 256) % 3;
      float v = 0.f;
#pragma unroll
      for (int ww = 0; ww < 8; ++ww) v += red_s[ww][ti][k];
      ts[ti][k] = v;
    }
    __syncthreads();
    if (tid < 16) {
      const int tt = tile * 16 + tid;
      const float S00 = ts[tid][0], S11 = ts[tid][1], S01 = ts[tid][2];
      const float inv = 1.0f / sqrtf((S00 + S11) / (float)C2 + a.eps);
      float l[8], m[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) l[jj] = (tl[tid][jj] + tl[tid][jj + 8]) * inv + a.b[jj];
      mhc_maps_from_logits(l, a.iters, m);
      if (tt < a.T) {
        float* mo = a.maps_out + (size_t)tt * 8;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) mo[jj] = m[jj];
      }
      const float ssin = m[0] * m[0] * S00 + 2.f * m[0] * m[1] * S01 + m[1] * m[1] * S11;
      mp[tid][0] = m[0];
      mp[tid][1] = m[1];
      mp[tid][2] = 1.0f / sqrtf(fmaxf(ssin, 0.f) / (float)C + a.eps);
    }
    __syncthreads();
    if (tv) {
      const float q0 = mp[li][0], q1 = mp[li][1], iv = mp[li][2];
#pragma unroll
      for (int j = 0; j < NSMAX; ++j) {
        if (j < NS) {
          const int cb = w * CW + 32 * j + 8 * g;
          float gm[8], o[8];
          ld8(a.gamma + cb, gm);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t wa = xs0[j][e >> 1], wb = xs1[j][e >> 1];
            const float x0 = __uint_as_float((e & 1) ? (wa & 0xFFFF0000u) : (wa << 16));
            const float x1 = __uint_as_float((e & 1) ? (wb & 0xFFFF0000u) : (wb << 16));
            o[e] = gm[e] * (q0 * x0 + q1 * x1) * iv;
          }
          st8(u + (size_t)t * C + cb, o);
        }
      }
    }
    __syncthreads();    // LDS reuse by the next tile
  }
}

hipError_t mhc(const MhcArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.C % 8 || a.C / 8 > 512) return hipErrorInvalidValue;
  // 16-token tiles on the matrix cores pay off once there are enough tiles;
  // decode-sized calls split the channels over waves (below); otherwise one
  // workgroup per token with W in registers
  // (C % 512: a wave's channel range, C / 8, is a whole number of two-step
  // load groups of 32 channels; at C = 256 a group would reach into the next
  // wave's channels and count them twice)
  if (a.dt == DT_BF16 && a.mode != MHC_EXIT && a.C % 512 == 0 && a.wsplit && a.T >= MHC_MFMA_MIN_T) {
    if (a.yp.part) return hipErrorInvalidValue;   // the tiled path reads y itself
    if (!a.wsplit_ready) {
      const int n = 8 * 2 * a.C;
      mhc_split_w<<<(n + 255) / 256, 256, 0, s>>>(a.w, a.wsplit, n);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const int ntiles = (a.T + 15) / 16;
    // Persistent grid: exactly the resident workgroups (a second wave of
    // workgroups would start only after the first finished its tiles), then
    // shrunk so that every workgroup gets the same number of tiles.
    static int per_cu = 0;
    if (per_cu == 0) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mhc_mfma_kernel, 512, 0) != hipSuccess || n < 1) n = 1;
      per_cu = n;
    }
    const int cu = device_cu_count();
    int grid = per_cu * (cu > 0 ? cu : 256);
    if (grid > ntiles) grid = ntiles;
    const int per_wg = (ntiles + grid - 1) / grid;
    grid = (ntiles + per_wg - 1) / per_wg;
    mhc_mfma_kernel<<<grid, 512, 0, s>>>(a, a.wsplit);
    return hipGetLastError();
  }
  // few tokens: one wave per (512-channel slice, token), partial sums in the scratch
  if (a.mode != MHC_EXIT && a.C % MHC_SLICE == 0 && a.T <= 64 && a.wsplit) {
    float* part = (float*)a.wsplit;     // T * (C / 512) * 11 floats <= 24 * 2C bf16 for T <= 64
    const dim3 grid(a.C / MHC_SLICE, a.T);
    if (a.dt == DT_BF16) {
      mhc_slice_a<bf16_t><<<grid, 64, 0, s>>>(a, part);
      mhc_slice_b<bf16_t><<<grid, 64, 0, s>>>(a, part);
    } else {
      mhc_slice_a<float><<<grid, 64, 0, s>>>(a, part);
      mhc_slice_b<float><<<grid, 64, 0, s>>>(a, part);
    }
    return hipGetLastError();
  }
  const int nv = a.C / 8;
  const int threads = ((nv + 63) / 64) * 64;
  int grid = a.grid > 0 ? a.grid : a.T;
  if (grid > a.T) grid = a.T;
  if (a.dt == DT_BF16)
    mhc_kernel<bf16_t><<<grid, threads, 0, s>>>(a);
  else
    mhc_kernel<float><<<grid, threads, 0, s>>>(a);
  return hipGetLastError();
}

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

}  // namespace lk
