// Causal softmax attention with grouped KV heads over a per-(layer, pass) KV
// cache slot.  Cache layout: K [B][Hkv][S_max][d], V transposed [B][Hkv][d][S_max],
// so that both operands of both products are read with the contraction axis
// contiguous.
//
// * attn_prefill_dma (bf16, d = 128, Hq / Hkv in 1, 2, 4, 8): flash-style.
//   One workgroup of eight waves per (256 / G queries, KV head, sequence);
//   the G heads of a group and 8 / G query blocks of 32 share every K / V^T
//   tile, which global -> LDS DMA brings in three tiles ahead.  Scores are
//   computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16), which leaves
//   each lane with one query column; the probabilities feed O^T = V^T P^T
//   directly from registers.  Online softmax in fp32 (base 2).
// * attn_decode_mfma (bf16, d = 128, up to 16 query columns = heads x new
//   tokens): eight waves per (split, KV head, sequence), splits only as many
//   as needed to fill the device, v_mfma_f32_16x16x32_bf16, operands read
//   straight from the cache; a combine kernel when there are several splits.
// * attn_f32: plain kernel for the fp32 configuration.
#include "common.h"
#include "kernels.h"

namespace lk {

constexpr float LOG2E = 1.4426950408889634f;

// ------------------------------------------------------------------ prefill, bf16
constexpr int PK = 64;    // keys per tile
constexpr int PD = 128;   // head dim

// ------------------------------------------------------------------ prefill, bf16, DMA
// Eight waves per workgroup: wave w serves query head kvh*G + w % G for the
// query sub-block w / G (32 queries), so one K / V^T tile in LDS serves
// 32 * 8 / G queries of each of the G heads.  Tiles move global -> LDS with
// global_load_lds_dwordx4 into a ring of four stages, three tiles ahead.
// LDS layouts (16-byte units, swizzled against the 64 banks):
//   K   [64 keys][128 d]:  unit c of row r at c ^ (r & 15)
//   V^T [128 d][64 keys]:  unit u (keys 8u .. 8u + 7) of row r at u ^ ((r >> 1) & 7)
// The score MFMA takes its K rows in the order kappa(rho), which swaps bits 2
// and 3 of the row index, so that a lane's probabilities for PV step mm are the
// eight consecutive keys 16 mm + 8 h .. + 7: one 16-byte read of V^T.
constexpr int AQ_STAGE = 2 * PK * PD;          // elements per stage (K + V^T, 32 KB)

DEV int kq_sw(int r, int c) { return r * PD + ((c ^ (r & 15)) << 3); }
DEV int vq_sw(int r, int u) { return r * PK + ((u ^ ((r >> 1) & 7)) << 3); }

constexpr int AQ_NW = 8;                       // waves per workgroup
constexpr int AQ_NS = 4;                       // LDS stages
constexpr int AQ_LDS = AQ_NS * AQ_STAGE * 2;   // 128 KB

__global__ __launch_bounds__(64 * AQ_NW, 1) void attn_prefill_dma(AttnArgs a) {
  constexpr int NW = AQ_NW, AHEAD = AQ_NS - 1;
  extern __shared__ __align__(16) bf16_t smem[];
  constexpr int NB = 16 / NW;                  // DMA blocks per wave per operand and tile
  const int G = a.Hq / a.Hkv;                  // 1, 2, 4 or 8
  const int QS = NW / G;                       // query sub-blocks per workgroup
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qb = gridDim.x - 1 - blockIdx.x;   // long rows first
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int j = kvh * G + wid % G;
  const int q0 = qb * 32 * QS + (wid / G) * 32; // this wave's first query
  const int h = lane >> 5, col = lane & 31;
  const int m = q0 + col;
  const bool qvalid = m < a.S_call;
  const int qpos = a.pos0 + m;
  const int kv_end = a.pos0 + min((qb + 1) * 32 * QS, a.S_call);   // keys the workgroup needs
  const int ntiles = (kv_end + PK - 1) / PK;
  const int wave_last = a.pos0 + min(q0 + 31, a.S_call - 1);       // last key this wave can see

  const bf16_t* Q = (const bf16_t*)a.q + (size_t)(b * a.S_call + min(m, a.S_call - 1)) * a.ldq + j * PD;
  bf16x8_t qf[8];
#pragma unroll
  for (int ds = 0; ds < 8; ++ds) qf[ds] = as_bf16x8(ldv4(Q + ds * 16 + h * 8));

  const bf16_t* Kg = (const bf16_t*)a.kcache + ((size_t)(b * a.Hkv + kvh) * a.S_max) * PD;
  const bf16_t* Vg = (const bf16_t*)a.vcache + ((size_t)(b * a.Hkv + kvh) * PD) * a.S_max;
  // DMA: per tile 16 K blocks of 4 rows and 16 V^T blocks of 8 rows; wave w
  // issues blocks 2w and 2w + 1 of each.  Lane l writes LDS bytes 16 l .. of
  // the block, so it fetches the global unit that the swizzle puts there.
  int koff[NB], voff[NB], kl[NB], vl[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int blk = NB * wid + i;
    const int kr = 4 * blk + (lane >> 4), ks = lane & 15;
    koff[i] = kr * PD + ((ks ^ (kr & 15)) << 3);
    kl[i] = blk * 512;
    const int vr = 8 * blk + (lane >> 3), vs = lane & 7;
    voff[i] = vr * a.S_max + ((vs ^ ((vr >> 1) & 7)) << 3);
    vl[i] = PK * PD + blk * 512;
  }
  auto issue = [&](int kt) {
    bf16_t* st = smem + (kt % AQ_NS) * AQ_STAGE;
    const int k0 = min(kt, ntiles - 1) * PK;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(Kg + (size_t)k0 * PD + koff[i]),
                                       (void __attribute__((address_space(3)))*)(st + kl[i]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(Vg + k0 + voff[i]),
                                       (void __attribute__((address_space(3)))*)(st + vl[i]), 16, 0, 0);
    }
  };
  auto sync = [&]() {
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;
  const float sc = LOG2E / sqrtf((float)PD);
  // MFMA row rho of the score block reads K row kappa(rho) (bits 2 and 3 swapped)
  const int krow = (col & 0x13) | ((col & 4) << 1) | ((col & 8) >> 1);

  static_assert(AQ_NS == 4 && NW == 8 && NB == 2, "wait counts below");
  // Software pipeline: the score MFMAs of tile kt + 1 are issued before the
  // softmax and PV of tile kt, so the softmax VALU work runs while they execute.
  // The two waves of a SIMD reach the same phase together after each barrier;
  // a wave raises its issue priority for its score MFMAs (and keeps a middle
  // one through softmax and PV), so the SIMD's other wave fills the VALU
  // slots rather than both waves alternating instruction by instruction
  // (measured: 3% over equal priorities; results are unchanged).
  f32x16_t sa[2], sb[2];                     // scores of the current / next tile
  // The two 32-key blocks alternate, so consecutive MFMAs are independent;
  // the K fragments of chunk ds + SA are read while the MFMAs of chunk ds
  // run (scheduling walls keep that order), so the MFMAs do not wait on the
  // LDS latency.
  constexpr int SA = 2;
  auto scores = [&](int kt, f32x16_t (&st)[2]) {
    const bf16_t* ks = smem + (kt % AQ_NS) * AQ_STAGE;
    bf16x8_t kf[SA + 1][2];
#pragma unroll
    for (int ds = 0; ds < SA; ++ds)
#pragma unroll
      for (int c = 0; c < 2; ++c) kf[ds][c] = as_bf16x8(ldv4(ks + kq_sw(c * 32 + krow, ds * 2 + h)));
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      if (ds + SA < 8) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
          kf[(ds + SA) % (SA + 1)][c] = as_bf16x8(ldv4(ks + kq_sw(c * 32 + krow, (ds + SA) * 2 + h)));
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) st[c] = mfma32(kf[ds % (SA + 1)][c], qf[ds], ds == 0 ? f32x16_t{} : st[c]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto softmax_pv = [&](int kt, f32x16_t (&st)[2]) {
    const bf16_t* vs = smem + (kt % AQ_NS) * AQ_STAGE + PK * PD;
    // st[c][r]: key kt*64 + 32c + 16(r/8) + 8h + r%8, query column `col`
    const bool diag = kt * PK + PK - 1 > a.pos0 + q0;
    float tmax = -INFINITY;
    if (diag) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * PK + c * 32 + (r >> 3) * 16 + h * 8 + (r & 7);
          const float v = (key <= qpos && key < kv_end) ? st[c][r] : -INFINITY;
          st[c][r] = v;
          tmax = fmaxf(tmax, v);
        }
    } else {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, st[c][r]);
    }
    tmax = x32_max(tmax) * sc;     // scaled (base-2) units
    // the running max moves only when the tile's max exceeds it by more than
    // 8: the probabilities stay below 2^8 and the result is the same softmax,
    // with fewer rescales of O
    const float mnew = tmax > mrun + 8.f ? tmax : mrun;
    const float mfin = (mnew == -INFINITY) ? 0.f : mnew;
    float psum = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_hw(fmaf(st[c][r], sc, -mfin));
        st[c][r] = p;
        psum += p;
      }
    if (__any(mnew > mrun)) {
      const float alpha = (mnew == -INFINITY) ? 1.f : exp2_hw(mrun - mnew);
      lrun *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    lrun += psum;
    mrun = mnew;
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      const int c = mm >> 1, half = mm & 1;
      uint32_t pw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pw[e] = pack_bf16x2(st[c][half * 8 + 2 * e], st[c][half * 8 + 2 * e + 1]);
      const bf16x8_t pf = as_bf16x8(u32x4_t{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8_t vf = as_bf16x8(ldv4(vs + vq_sw(db * 32 + col, 2 * mm + h)));
        o[db] = mfma32(vf, pf, o[db]);
      }
    }
  };
  // keys kv_end .. of the last tile hold arbitrary bits: clear V^T there once
  // the tile has landed, before any PV reads it (probabilities there are 0,
  // but 0 * NaN would not be)
  auto mask_tail = [&]() {
    const int kt = ntiles - 1;
    bf16_t* vs = smem + (kt % AQ_NS) * AQ_STAGE + PK * PD;
    const int lim = kv_end - kt * PK;
    for (int idx = tid; idx < PD * 8; idx += 64 * NW) {
      const int r = idx >> 3, u = idx & 7;
      if (8 * u + 8 > lim) {
        bf16_t* p = vs + vq_sw(r, u);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (8 * u + e >= lim) p[e] = 0;
      }
    }
  };
  const bool ragged = kv_end % PK != 0;
  for (int t = 0; t < AHEAD; ++t) issue(t);
  asm volatile("s_waitcnt vmcnt(8)" ::: "memory");    // tile 0 (4 loads) landed, tiles 1, 2 in flight
  sync();
  if (ntiles == 1 && ragged) { mask_tail(); sync(); }
  scores(0, sa);
  for (int kt = 0; kt < ntiles; kt += 2) {
    // even step: scores of kt + 1 into sb, softmax / PV of kt from sa
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");  // tile kt + 1 landed (tile kt + 2 may be in flight)
    sync();
    issue(kt + AHEAD);                       // into the stage of tile kt - 1, finished before this barrier
    if (kt + 1 == ntiles - 1 && ragged) mask_tail();   // ordered before its PV by the next barrier
    __builtin_amdgcn_s_setprio(2);
    if ((kt + 1) * PK <= wave_last) scores(kt + 1, sb);   // wave-uniform: tiles past the
    __builtin_amdgcn_s_setprio(1);
    if (kt * PK <= wave_last) softmax_pv(kt, sa);           // wave's last query are skipped
    __builtin_amdgcn_s_setprio(0);
    if (kt + 1 >= ntiles) break;
    // odd step: scores of kt + 2 into sa, softmax / PV of kt + 1 from sb
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    sync();
    issue(kt + 1 + AHEAD);
    if (kt + 2 == ntiles - 1 && ragged) mask_tail();
    __builtin_amdgcn_s_setprio(2);
    if ((kt + 2) * PK <= wave_last) scores(kt + 2, sa);
    __builtin_amdgcn_s_setprio(1);
    if ((kt + 1) * PK <= wave_last) softmax_pv(kt + 1, sb);
    __builtin_amdgcn_s_setprio(0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load may still target LDS at exit
  if (qvalid) {
    const float ltot = x32_sum(lrun);
    const float inv = 1.0f / ltot;
    bf16_t* O = (bf16_t*)a.out + (size_t)(b * a.S_call + m) * a.ldo + j * PD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + g4 * 8 + h * 4;
        const uint32_t w0 = pack_bf16x2(o[db][g4 * 4] * inv, o[db][g4 * 4 + 1] * inv);
        const uint32_t w1 = pack_bf16x2(o[db][g4 * 4 + 2] * inv, o[db][g4 * 4 + 3] * inv);
        *(u32x2_t*)(O + d0) = u32x2_t{w0, w1};
      }
  }
}

// ------------------------------------------------------------------ decode, bf16
// One workgroup of DW waves per (split, KV head, sequence); wave w takes the
// 64-key rounds w, w + DW, ... of the split, so the waves stream neighbouring
// cache lines together.  Query columns c < ncol are (token t = c / G, head
// kvh*G + c % G).  A round loads its K rows and its V^T columns at once
// (32 KB per wave in flight), then computes four S^T blocks of 16 keys whose
// rows are ordered so that, for PV step kk, lane group g holds the
// probabilities of keys 32kk + 8g + 0..7, matching a contiguous 16-byte read
// of V^T.  The waves' (max, sum, O) are merged in LDS by a fixed tree
// (w + 4 into w, then w + 2, then w + 1).  A single split writes the output;
// several splits write fp32 partials for attn_combine.
constexpr int DW = 8;

DecodePlan decode_plan(int B, int Hkv, int kv_len, int cu) {
  DecodePlan p{};
  const int groups = B * Hkv > 0 ? B * Hkv : 1;
  int want = (cu + groups - 1) / groups;
  if (want < 1) want = 1;
  int len = (kv_len + want - 1) / want;
  len = (len + 63) / 64 * 64;
  if (len < 64) len = 64;
  p.split_len = len;
  p.n_split = (kv_len + len - 1) / len;
  return p;
}

int decode_max_splits(int B, int Hkv, int S_max, int cu) {
  const int groups = B * Hkv > 0 ? B * Hkv : 1;
  const int want = (cu + groups - 1) / groups;
  const int cap = (S_max + 63) / 64;
  return want < 1 ? 1 : (want < cap ? want : cap);
}

__global__ __launch_bounds__(64 * DW) void attn_decode_mfma(AttnArgs a) {
  __shared__ float mrg[DW / 2][16][PD + 2];   // o[0..127], max, sum per column
  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int ncol = G * a.S_call;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const bool cvalid = c < ncol;
  const int tq = cvalid ? c / G : 0, jq = kvh * G + (cvalid ? c % G : 0);
  const int pos0 = a.pos_dev ? min(max(a.pos_dev[b], 0), a.pos0) : a.pos0;   // this sequence's first new position
  const int kv_len = pos0 + a.S_call;              // keys [0, kv_len) exist
  const int lim = pos0 + tq + 1;                   // visible to this column
  const int k_begin = s * a.split_len;
  const int k_end = min(k_begin + a.split_len, kv_len);

  const bf16_t* Q = (const bf16_t*)a.q + (size_t)(b * a.S_call + tq) * a.ldq + jq * PD;
  bf16x8_t qf[4];
  const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) qf[ds] = as_bf16x8(cvalid ? ldv4(Q + ds * 32 + g * 8) : zero);

  const bf16_t* Kg = (const bf16_t*)a.kcache + ((size_t)(b * a.Hkv + kvh) * a.S_max) * PD;
  const bf16_t* Vg = (const bf16_t*)a.vcache + ((size_t)(b * a.Hkv + kvh) * PD) * a.S_max;
  const float sc = LOG2E / sqrtf((float)PD);

  f32x4_t o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;

  for (int k0 = k_begin + wid * 64; k0 < k_end; k0 += DW * 64) {
    // loads of the whole round first: K rows (S^T operand) and V^T (PV operand).
    // Keys past k_end stay inside the slot (S_max % 64 == 0) and are masked.
    u32x4_t kf[4][4], vf[2][8];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const int key = k0 + 32 * (sb >> 1) + (c >> 2) * 8 + (sb & 1) * 4 + (c & 3);
      const bf16_t* kr = Kg + (size_t)key * PD + g * 8;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) kf[sb][ds] = ldv4(kr + ds * 32);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int db = 0; db < 8; ++db) vf[kk][db] = ldv4(Vg + (size_t)(db * 16 + c) * a.S_max + k0 + 32 * kk + 8 * g);

    f32x4_t st[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      st[sb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) st[sb] = mfma16(as_bf16x8(kf[sb][ds]), qf[ds], st[sb]);
    }
    // st[sb][i]: column c, key k0 + 32*(sb/2) + 8g + 4*(sb%2) + i
    float tmax = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 32 * (sb >> 1) + 8 * g + 4 * (sb & 1) + i;
        const float v = (key < lim && key < k_end) ? st[sb][i] * sc : -INFINITY;
        st[sb][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = x32_max(x16_max(tmax));
    const float mnew = fmaxf(mrun, tmax);
    const float alpha = (mnew == -INFINITY) ? 1.f : exp2_hw(mrun - mnew);
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = (mnew == -INFINITY) ? 0.f : exp2_hw(st[sb][i] - mnew);
        st[sb][i] = p;
        psum += p;
      }
    lrun = lrun * alpha + psum;
    mrun = mnew;
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] *= alpha;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t pw[4];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        pw[e] = pack_bf16x2(st[2 * kk][2 * e], st[2 * kk][2 * e + 1]);
        pw[2 + e] = pack_bf16x2(st[2 * kk + 1][2 * e], st[2 * kk + 1][2 * e + 1]);
      }
      // probabilities of masked keys are exactly 0, but V there may hold any
      // bits (a NaN pattern would poison 0 * v): clear V past the end
      const bf16x8_t pf = as_bf16x8(u32x4_t{pw[0], pw[1], pw[2], pw[3]});
      const int key0 = k0 + 32 * kk + 8 * g;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        u32x4_t v = vf[kk][db];
        if (key0 + 8 > k_end) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (key0 + e >= k_end) v[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        }
        o[db] = mfma16(as_bf16x8(v), pf, o[db]);
      }
    }
  }
  // full row sum of a column (its four lane groups)
  float ltot = x32_sum(x16_sum(lrun));

  // merge waves: step h = 4, 2, 1: waves [h, 2h) hand their state to w - h
  for (int h = DW / 2; h >= 1; h >>= 1) {
    if (wid >= h && wid < 2 * h) {
      float* slot = &mrg[wid - h][c][0];
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) slot[db * 16 + g * 4 + i] = o[db][i];
      if (g == 0) { slot[PD] = mrun; slot[PD + 1] = ltot; }
    }
    __syncthreads();
    if (wid < h) {
      const float* slot = &mrg[wid][c][0];
      const float m2 = slot[PD], l2 = slot[PD + 1];
      const float M = fmaxf(mrun, m2);
      const float a1 = (mrun == -INFINITY) ? 0.f : exp2_hw(mrun - M);
      const float a2 = (m2 == -INFINITY) ? 0.f : exp2_hw(m2 - M);
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[db][i] = o[db][i] * a1 + slot[db * 16 + g * 4 + i] * a2;
      ltot = ltot * a1 + l2 * a2;
      mrun = M;
    }
    __syncthreads();
  }
  if (wid != 0 || !cvalid) return;
  if (a.n_split == 1) {
    const float inv = 1.f / ltot;
    bf16_t* O = (bf16_t*)a.out + (size_t)(b * a.S_call + tq) * a.ldo + jq * PD;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint32_t w0 = pack_bf16x2(o[db][0] * inv, o[db][1] * inv);
      const uint32_t w1 = pack_bf16x2(o[db][2] * inv, o[db][3] * inv);
      *(u32x2_t*)(O + db * 16 + g * 4) = u32x2_t{w0, w1};
    }
    return;
  }
  float* P = a.part + ((((size_t)(b * a.S_call + tq) * a.Hq + jq) * a.n_split) + s) * (PD + 2);
#pragma unroll
  for (int db = 0; db < 8; ++db)
    *(float4*)(P + db * 16 + g * 4) = make_float4(o[db][0], o[db][1], o[db][2], o[db][3]);
  if (g == 0) { P[PD] = mrun; P[PD + 1] = ltot; }
}

// out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M)
template <typename T>
__global__ __launch_bounds__(128) void attn_combine(AttnArgs a) {
  const int row = blockIdx.x;                   // (b * S_call + t) * Hq + j
  const int dd = threadIdx.x;
  const float* P = a.part + (size_t)row * a.n_split * (a.d + 2);
  float M = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, P[s * (a.d + 2) + a.d]);
  float L = 0.f, acc = 0.f;
  for (int s = 0; s < a.n_split; ++s) {
    const float ms = P[s * (a.d + 2) + a.d];
    const float w = (ms == -INFINITY) ? 0.f : exp2_hw(ms - M);
    L += P[s * (a.d + 2) + a.d + 1] * w;
    if (dd < a.d) acc += P[s * (a.d + 2) + dd] * w;
  }
  const int tok = row / a.Hq, j = row % a.Hq;
  if (dd < a.d) st1((T*)a.out + (size_t)tok * a.ldo + j * a.d + dd, acc / L);
}

// ------------------------------------------------------------------ fp32
// One thread per (query, head); keys in order; online softmax.  Writes either
// the final output (n_split == 0) or split partials in the decode layout.
template <int D>
__global__ __launch_bounds__(64) void attn_f32(AttnArgs a) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  const int j = blockIdx.y, b = blockIdx.z;
  if (t >= a.S_call) return;
  const int G = a.Hq / a.Hkv, kvh = j / G;
  const float* q = (const float*)a.q + (size_t)(b * a.S_call + t) * a.ldq + j * D;
  const float* K = (const float*)a.kcache + ((size_t)(b * a.Hkv + kvh) * a.S_max) * D;
  const float* V = (const float*)a.vcache + ((size_t)(b * a.Hkv + kvh) * D) * a.S_max;
  float qr[D], o[D];
  const float sc = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int i = 0; i < D; ++i) { qr[i] = q[i]; o[i] = 0.f; }
  float m = -INFINITY, l = 0.f;
  const int last = (a.pos_dev ? min(max(a.pos_dev[b], 0), a.pos0) : a.pos0) + t;
  for (int key = 0; key <= last; ++key) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) s += qr[i] * K[(size_t)key * D + i];
    s *= sc;
    const float mn = fmaxf(m, s);
    const float al = expf(m - mn), p = expf(s - mn);
    l = l * al + p;
#pragma unroll
    for (int i = 0; i < D; ++i) o[i] = o[i] * al + p * V[(size_t)i * a.S_max + key];
    m = mn;
  }
  float* out = (float*)a.out + (size_t)(b * a.S_call + t) * a.ldo + j * D;
#pragma unroll
  for (int i = 0; i < D; ++i) out[i] = o[i] / l;
}

static hipError_t launch_f32(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.S_call + 63) / 64, a.Hq, a.B);
  if (a.d == 64) attn_f32<64><<<grid, 64, 0, s>>>(a);
  else if (a.d == 128) attn_f32<128><<<grid, 64, 0, s>>>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t attn_prefill(const AttnArgs& a, hipStream_t s) {
  if (a.S_call <= 0 || a.B <= 0) return hipSuccess;
  if (a.dt == DT_F32) return launch_f32(a, s);
  if (a.pos_dev) return hipErrorInvalidValue;   // one start position per call
  const int G = a.Hq / a.Hkv;
  if (a.d != PD || a.Hq % a.Hkv || !(G == 1 || G == 2 || G == 4 || G == 8) || a.S_max % 64)
    return hipErrorInvalidValue;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_prefill_dma, hipFuncAttributeMaxDynamicSharedMemorySize, AQ_LDS);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int qpw = 32 * (AQ_NW / G);   // queries per workgroup
  dim3 grid((a.S_call + qpw - 1) / qpw, a.Hkv, a.B);
  attn_prefill_dma<<<grid, 64 * AQ_NW, AQ_LDS, s>>>(a);
  return hipGetLastError();
}

hipError_t attn_decode(const AttnArgs& a, hipStream_t s) {
  if (a.S_call <= 0 || a.B <= 0) return hipSuccess;
  if (a.dt == DT_F32) return launch_f32(a, s);
  const int G = a.Hq / a.Hkv;
  if (a.d != PD || a.Hq % a.Hkv || G * a.S_call > 16 || a.S_max % 64 || a.split_len % 64) return hipErrorInvalidValue;
  const int kv_len = a.pos0 + a.S_call;
  if ((long)a.n_split * a.split_len < kv_len) return hipErrorInvalidValue;
  dim3 grid(a.n_split, a.Hkv, a.B);
  attn_decode_mfma<<<grid, 64 * DW, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  attn_combine<bf16_t><<<a.B * a.S_call * a.Hq, 128, 0, s>>>(a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ KV append
// Writes the K and V columns of B q|k|v rows (one new position per sequence,
// already rounded to the storage type) at position `pos` of a cache slot,
// K [B][Hkv][S_max][d] and V^T [B][Hkv][d][S_max]: the same values the fused
// QKV epilogue stores, for callers whose projection covered several slots.
template <typename T>
__global__ __launch_bounds__(256) void kv_append_kernel(const T* __restrict__ qkv, long ld, int q_cols, int B,
                                                        int Hkv, int d, T* __restrict__ kc, T* __restrict__ vc,
                                                        int S_max, int pos) {
  const int n = B * Hkv * d;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    const int b = i / (Hkv * d), r = i - b * Hkv * d, hk = r / d, dd = r - hk * d;
    const T* row = qkv + (size_t)b * ld + q_cols;
    kc[(((size_t)b * Hkv + hk) * S_max + pos) * d + dd] = row[hk * d + dd];
    vc[(((size_t)b * Hkv + hk) * d + dd) * S_max + pos] = row[Hkv * d + hk * d + dd];
  }
}

hipError_t kv_append(int dt, const void* qkv, long ld, int q_cols, int B, int Hkv, int d, void* kcache,
                     void* vcache, int S_max, int pos, hipStream_t s) {
  const int n = B * Hkv * d;
  if (n <= 0) return hipSuccess;
  const int grid = (n + 255) / 256;
  if (dt == DT_BF16)
    kv_append_kernel<bf16_t><<<grid, 256, 0, s>>>((const bf16_t*)qkv, ld, q_cols, B, Hkv, d, (bf16_t*)kcache,
                                                  (bf16_t*)vcache, S_max, pos);
  else
    kv_append_kernel<float><<<grid, 256, 0, s>>>((const float*)qkv, ld, q_cols, B, Hkv, d, (float*)kcache,
                                                 (float*)vcache, S_max, pos);
  return hipGetLastError();
}

}  // namespace lk
