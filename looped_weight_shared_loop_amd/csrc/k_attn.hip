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
// * attn_prefill_d256 (bf16, d = 256, Hq / Hkv in 1, 2, 4): the same scheme
//   with four waves (one per SIMD), two-stage K and V^T rings.
// * attn_decode_mfma<D> (bf16, d = 128 or 256, up to 16 query columns =
//   heads x new tokens): eight waves per (split, KV head, sequence), splits
//   only as many as needed to fill the device, v_mfma_f32_16x16x32_bf16,
//   operands read straight from the cache; a combine kernel when there are
//   several splits.
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
constexpr int AQ_LDS_MAX = 160 * 1024;          // the CU's LDS: with a paged cache, up to 8,192 tile pages

__global__ __launch_bounds__(64 * AQ_NW, 1) void attn_prefill_dma(AttnArgs a) {
  constexpr int NW = AQ_NW, AHEAD = AQ_NS - 1;
  extern __shared__ __align__(16) bf16_t smem[];
  constexpr int NB = 16 / NW;                  // DMA blocks per wave per operand and tile
  const int G = a.Hq / a.Hkv;                  // 1, 2, 4 or 8
  const int QS = NW / G;                       // query sub-blocks per workgroup
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  // query blocks slowest in the dispatch order, longest first: every KV head's
  // long rows start before any short ones, and with one sequence workgroup n
  // serves KV head n % Hkv (the XCD a workgroup lands on follows n % 8)
  const int qb = gridDim.z - 1 - blockIdx.z;
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int j = kvh * G + wid % G;
  const int q0 = qb * 32 * QS + (wid / G) * 32; // this wave's first query
  const int h = lane >> 5, col = lane & 31;
  const int m = q0 + col;
  const bool qvalid = m < a.S_call;
  const int qpos = a.pos0 + m;
  const int kv_end = a.pos0 + min((qb + 1) * 32 * QS, a.S_call);   // keys the workgroup needs
  const int ntiles = (kv_end + PK - 1) / PK;
  const int wave_last = a.pos0 + min(q0 + 31, a.S_call - 1);       // last key this wave can see

  // paged cache: the page of every tile the workgroup reads, kept in LDS past the ring
  const bool paged = a.pages.table != nullptr;
  int* pglist = reinterpret_cast<int*>(smem + AQ_NS * AQ_STAGE);
  if (paged) {
    for (int t = tid; t < ntiles; t += 64 * NW) pglist[t] = kv_page(a.pages, b, t * PK);
    __syncthreads();
  }

  const bf16_t* Q = (const bf16_t*)a.q + (size_t)(b * a.S_call + min(m, a.S_call - 1)) * a.ldq + j * PD;
  bf16x8_t qf[8];
#pragma unroll
  for (int ds = 0; ds < 8; ++ds) qf[ds] = as_bf16x8(ldv4(Q + ds * 16 + h * 8));

  const bf16_t* Kg = (const bf16_t*)a.kcache + (paged ? 0 : ((size_t)(b * a.Hkv + kvh) * a.S_max) * PD);
  const bf16_t* Vg = (const bf16_t*)a.vcache + (paged ? 0 : ((size_t)(b * a.Hkv + kvh) * PD) * a.S_max);
  const int vstride = kv_vstride(a.pages, a.S_max);
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
    voff[i] = vr * vstride + ((vs ^ ((vr >> 1) & 7)) << 3);
    vl[i] = PK * PD + blk * 512;
  }
  auto issue = [&](int kt) {
    bf16_t* st = smem + (kt % AQ_NS) * AQ_STAGE;
    const int tile = min(kt, ntiles - 1);
    const bf16_t* Kt;
    const bf16_t* Vt;
    if (paged) {
      const int pg = __builtin_amdgcn_readfirstlane(pglist[tile]);
      Kt = Kg + (((size_t)pg * a.Hkv + kvh) * KV_PAGE) * PD;
      Vt = Vg + ((size_t)pg * a.Hkv + kvh) * PD * KV_PAGE;
    } else {
      Kt = Kg + (size_t)tile * PK * PD;
      Vt = Vg + tile * PK;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(Kt + koff[i]),
                                       (void __attribute__((address_space(3)))*)(st + kl[i]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(Vt + voff[i]),
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
    auto mask = [&]() {
      if (diag) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt * PK + c * 32 + (r >> 3) * 16 + h * 8 + (r & 7);
            if (!(key <= qpos && key < kv_end)) st[c][r] = -INFINITY;
          }
      }
    };
    mask();
    // Probabilities against the running max, without the tile's own max:
    // bf16 keeps its relative precision at any magnitude, so p may grow far
    // past 1 before anything is lost.  Only when a lane's partial sum passes
    // 2^64 (a score 64 past the running max in base-2 units; 2^64 times 2^18
    // keys stays far inside float32), and at tile 0, where there is no running
    // max yet, is the tile's max taken: from the scores recomputed out of the
    // K tile, which is still in LDS.  Four independent partial sums (and maxima
    // below), so that a wave alone on its SIMD's vector ALU is not held up by
    // one dependent chain.
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
    bool slow = kt == 0;                   // every wave starts at tile 0
    if (!slow) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_hw(fmaf(st[c][r], sc, -mrun));
          st[c][r] = p;
          ps[r & 3] += p;
        }
      slow = __any(!((ps[0] + ps[1]) + (ps[2] + ps[3]) <= 0x1p64f));
    }
    float mnew = mrun;
    if (slow) {
      if (kt != 0) {
        scores(kt, st);
        mask();
      }
      float tm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) tm[r & 3] = fmaxf(tm[r & 3], st[c][r]);
      float tmax = fmaxf(fmaxf(tm[0], tm[1]), fmaxf(tm[2], tm[3]));
      tmax = x32_max(tmax) * sc;     // scaled (base-2) units
      // the running max moves only when the tile's max exceeds it by more
      // than 8, so O is rescaled rarely
      mnew = tmax > mrun + 8.f ? tmax : mrun;
      const float mfin = (mnew == -INFINITY) ? 0.f : mnew;
#pragma unroll
      for (int i = 0; i < 4; ++i) ps[i] = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_hw(fmaf(st[c][r], sc, -mfin));
          st[c][r] = p;
          ps[r & 3] += p;
        }
      if (__any(mnew > mrun)) {
        const float alpha = (mnew == -INFINITY) ? 1.f : exp2_hw(mrun - mnew);
        lrun *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
    }
    const float psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
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

// ------------------------------------------------------------------ prefill, bf16, d = 256
// Four waves per workgroup, one per SIMD: wave w serves query head kvh*G + w % G
// for the query sub-block w / G (32 queries), so one K / V^T tile of 64 keys
// serves 32 * 4 / G queries of each of the G heads (G in 1, 2, 4).  At d = 256
// a wave's O (32 queries x 256) takes 128 accumulators and its Q fragments 64
// registers: that fits only with a SIMD's whole register file, so there is no
// second wave on the SIMD to fill the vector ALU while the matrix core runs.
// Instead the wave itself overlaps them: the score MFMAs of tile kt + 1 are
// issued before the softmax of tile kt.  K and V^T live in separate rings of
// two 32 KB stages each (K of tiles kt + 1 and kt + 2, V^T of tiles kt and
// kt + 1), so the loads of one tile have a whole tile's work to land in.
// LDS layouts (16-byte units, swizzled against the 64 banks):
//   K   [64 keys][256 d]:  unit c (0..31) of row r at c ^ (r & 15)
//   V^T [256 d][64 keys]:  as for d = 128
// Scores use the same key permutation as the d = 128 kernel, and the score
// contraction runs as two 128-deep halves with their own accumulators (four
// independent chains per tile), summed before the softmax.
constexpr int PD2 = 256;
constexpr int A2_NW = 4;
constexpr int A2_KST = PK * PD2;                // elements per K stage (32 KB)
constexpr int A2_LDS = 4 * A2_KST * 2;          // two K stages + two V^T stages: 128 KB

DEV int kq2_sw(int r, int c) { return r * PD2 + ((c ^ (r & 15)) << 3); }

__global__ __launch_bounds__(64 * A2_NW, 1) void attn_prefill_d256(AttnArgs a) {
  constexpr int NW = A2_NW;
  constexpr int NB = 32 / NW;                  // DMA blocks of 1 KB per wave per operand and tile
  extern __shared__ __align__(16) bf16_t smem[];
  bf16_t* kring = smem;                        // [2][64][256]
  bf16_t* vring = smem + 2 * A2_KST;           // [2][256][64]
  const int G = a.Hq / a.Hkv;                  // 1, 2 or 4
  const int QS = NW / G;                       // query sub-blocks per workgroup
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  // query blocks slowest in the dispatch order, longest first: every KV head's
  // long rows start before any short ones, and with one sequence workgroup n
  // serves KV head n % Hkv (the XCD a workgroup lands on follows n % 8)
  const int qb = gridDim.z - 1 - blockIdx.z;
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int j = kvh * G + wid % G;
  const int q0 = qb * 32 * QS + (wid / G) * 32;
  const int h = lane >> 5, col = lane & 31;
  const int m = q0 + col;
  const bool qvalid = m < a.S_call;
  const int qpos = a.pos0 + m;
  const int kv_end = a.pos0 + min((qb + 1) * 32 * QS, a.S_call);
  const int ntiles = (kv_end + PK - 1) / PK;

  const bool paged = a.pages.table != nullptr;
  int* pglist = reinterpret_cast<int*>(smem + 4 * A2_KST);
  if (paged) {
    for (int t = tid; t < ntiles; t += 64 * NW) pglist[t] = kv_page(a.pages, b, t * PK);
    __syncthreads();
  }

  const bf16_t* Q = (const bf16_t*)a.q + (size_t)(b * a.S_call + min(m, a.S_call - 1)) * a.ldq + j * PD2;
  bf16x8_t qf[16];
#pragma unroll
  for (int ds = 0; ds < 16; ++ds) qf[ds] = as_bf16x8(ldv4(Q + ds * 16 + h * 8));
  // Register classes: O (128) and Q (64) live in the accumulation registers
  // (MFMA operands may come from there), leaving the vector registers to the
  // scores, the fragments and the softmax.  Everything that touches O is an
  // MFMA or the in-place rescale below, so the compiler keeps it there.
#pragma unroll
  for (int ds = 0; ds < 16; ++ds) asm volatile("" : "+a"(qf[ds]));

  const bf16_t* Kg = (const bf16_t*)a.kcache + (paged ? 0 : ((size_t)(b * a.Hkv + kvh) * a.S_max) * PD2);
  const bf16_t* Vg = (const bf16_t*)a.vcache + (paged ? 0 : ((size_t)(b * a.Hkv + kvh) * PD2) * a.S_max);
  const int vstride = kv_vstride(a.pages, a.S_max);
  // K: 32 blocks of 2 rows, V^T: 32 blocks of 8 rows; wave w issues blocks
  // NB w .. NB w + NB - 1 of each.  Lane l writes LDS bytes 16 l .. of the
  // block, so it fetches the global unit that the swizzle puts there.
  const int kr_l = lane >> 5, ks_l = lane & 31, vr_l = lane >> 3, vs_l = lane & 7;
  auto tile_src = [&](int tile, const bf16_t*& Kt, const bf16_t*& Vt) {
    if (paged) {
      const int pg = __builtin_amdgcn_readfirstlane(pglist[tile]);
      Kt = Kg + (((size_t)pg * a.Hkv + kvh) * KV_PAGE) * PD2;
      Vt = Vg + ((size_t)pg * a.Hkv + kvh) * PD2 * KV_PAGE;
    } else {
      Kt = Kg + (size_t)tile * PK * PD2;
      Vt = Vg + tile * PK;
    }
  };
  auto issue_k = [&](int kt) {
    const bf16_t *Kt, *Vt;
    tile_src(min(kt, ntiles - 1), Kt, Vt);
    bf16_t* st = kring + (kt & 1) * A2_KST;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int blk = NB * wid + i;
      const int kr = 2 * blk + kr_l;
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(Kt + kr * PD2 + ((ks_l ^ (kr & 15)) << 3)),
          (void __attribute__((address_space(3)))*)(st + blk * 512), 16, 0, 0);
    }
  };
  auto issue_v = [&](int kt) {
    const bf16_t *Kt, *Vt;
    tile_src(min(kt, ntiles - 1), Kt, Vt);
    bf16_t* st = vring + (kt & 1) * A2_KST;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int blk = NB * wid + i;
      const int vr = 8 * blk + vr_l;
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(Vt + (size_t)vr * vstride + ((vs_l ^ ((vr >> 1) & 7)) << 3)),
          (void __attribute__((address_space(3)))*)(st + blk * 512), 16, 0, 0);
    }
  };
  auto sync = [&]() {
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  f32x16_t o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
#pragma unroll
  for (int db = 0; db < 8; ++db) asm volatile("" : "+a"(o[db]));
  float mrun = -INFINITY, lrun = 0.f;
  const float sc = LOG2E / sqrtf((float)PD2);
  const int krow = (col & 0x13) | ((col & 4) << 1) | ((col & 8) >> 1);

  // LDS read addresses: only the swizzled part depends on the lane; the key
  // block, the d half, the O block and the stage are constant offsets, which
  // the reads take as immediates.  K unit 2 ds + h (+ 16 for the upper d half)
  // of row r = 32 c + krow sits at unit (2 ds + h) ^ (krow & 15); V^T unit
  // 2 mm + h of row 32 db + col at (2 mm + h) ^ ((col >> 1) & 7).
  const int kx = krow & 15, vy = (col >> 1) & 7;
  int kofs[8], vofs[4];
#pragma unroll
  for (int ds = 0; ds < 8; ++ds) kofs[ds] = krow * PD2 + (((2 * ds + h) ^ kx) << 3);
#pragma unroll
  for (int mm = 0; mm < 4; ++mm) vofs[mm] = col * PK + (((2 * mm + h) ^ vy) << 3);

  f32x16_t sa[2], sb[2];
  // With one wave per SIMD nothing else hides the LDS latency or fills the
  // vector ALU while the matrix core runs, so the wave interleaves its own
  // work: the K fragments of score step ds + 2 are read during step ds, and
  // the softmax of tile kt runs in eight slices between the eight score steps
  // of tile kt + 1 (scheduling walls keep each slice beside its MFMAs).
  bf16x8_t kf[3][4];
  auto ldk = [&](const bf16_t* ks, int ds, bf16x8_t (&f)[4]) {
    const bf16_t* kp = ks + kofs[ds];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f[2 * c] = as_bf16x8(ldv4(kp + c * 32 * PD2));
      f[2 * c + 1] = as_bf16x8(ldv4(kp + c * 32 * PD2 + 128));
    }
  };
  // one score step: MFMAs of chunk ds (and the reads of chunk ds + 2)
  auto score_step = [&](const bf16_t* ks, int ds, f32x16_t (&lo)[2], f32x16_t (&hi)[2]) {
    if (ds + 2 < 8) ldk(ks, ds + 2, kf[(ds + 2) % 3]);
    const bf16x8_t(&f)[4] = kf[ds % 3];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      lo[c] = mfma32(f[2 * c], qf[ds], ds == 0 ? f32x16_t{} : lo[c]);
      hi[c] = mfma32(f[2 * c + 1], qf[8 + ds], ds == 0 ? f32x16_t{} : hi[c]);
    }
  };
  auto scores = [&](int kstage, f32x16_t (&st)[2]) {
    const bf16_t* ks = kring + kstage * A2_KST;
    f32x16_t lo[2], hi[2];
    ldk(ks, 0, kf[0]);
    ldk(ks, 1, kf[1]);
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      score_step(ks, ds, lo, hi);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) st[c] = lo[c] + hi[c];
  };
  // the masked scores of a tile that reaches past the wave's first query
  auto mask_diag = [&](int kt, f32x16_t (&st)[2]) {
    if (kt * PK + PK - 1 > a.pos0 + q0) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * PK + c * 32 + (r >> 3) * 16 + h * 8 + (r & 7);
          if (!(key <= qpos && key < kv_end)) st[c][r] = -INFINITY;
        }
    }
  };
  // Scores of the next tile (nxt) fused with the softmax of this one (cur):
  // its probabilities pc against the running max, without the tile's own max
  // (bf16 keeps its relative precision at any magnitude).  Returns whether
  // some lane's partial sum passed 2^64 or is not finite (always at tile 0,
  // where the running max is -inf): then rescale_pv takes the tile's max from
  // the raw scores cur, which are kept for that.
  float pc[2][16];
  uint32_t pw[4][4];
  auto pack = [&](int mm) {
    const int c = mm >> 1, half = mm & 1;
#pragma unroll
    for (int e = 0; e < 4; ++e) pw[mm][e] = pack_bf16x2(pc[c][half * 8 + 2 * e], pc[c][half * 8 + 2 * e + 1]);
  };
  auto scores_softmax = [&](int kstage, f32x16_t (&nxt)[2], const f32x16_t (&cur)[2], float& psum) {
    const bf16_t* ks = kring + kstage * A2_KST;
    f32x16_t lo[2], hi[2];
    ldk(ks, 0, kf[0]);
    ldk(ks, 1, kf[1]);
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      score_step(ks, ds, lo, hi);
      if (ds < 4) {                     // eight probabilities per step
        const int c = ds >> 1, r0 = (ds & 1) * 8;
#pragma unroll
        for (int r = r0; r < r0 + 8; ++r) {
          const float p = exp2_hw(fmaf(cur[c][r], sc, -mrun));
          pc[c][r] = p;
          ps[r & 3] += p;
        }
        // formed here, beside this step's MFMAs (the compiler would otherwise
        // sink them to their uses after the rescale branch)
        asm volatile("" : "+v"(ps[0]), "+v"(ps[1]), "+v"(ps[2]), "+v"(ps[3]));
      } else if (ds < 6) {              // bf16 pairs for two PV steps
#pragma unroll
        for (int mm = 2 * (ds - 4); mm < 2 * (ds - 4) + 2; ++mm) {
          pack(mm);
          asm volatile("" : "+v"(pw[mm][0]), "+v"(pw[mm][1]), "+v"(pw[mm][2]), "+v"(pw[mm][3]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
#pragma unroll
    for (int c = 0; c < 2; ++c) nxt[c] = lo[c] + hi[c];
  };
  auto rescale_pv = [&](int vstage, const f32x16_t (&cur)[2], float psum) {
    const bf16_t* vs = vring + vstage * A2_KST;
    float mnew = mrun;
    if (__any(!(psum <= 0x1p64f))) {
      float tm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) tm[r & 3] = fmaxf(tm[r & 3], cur[c][r]);
      float tmax = fmaxf(fmaxf(tm[0], tm[1]), fmaxf(tm[2], tm[3]));
      tmax = x32_max(tmax) * sc;
      // lazy rescaling, as in the d = 128 kernel
      mnew = tmax > mrun + 8.f ? tmax : mrun;
      const float mfin = (mnew == -INFINITY) ? 0.f : mnew;
      float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_hw(fmaf(cur[c][r], sc, -mfin));
          pc[c][r] = p;
          ps[r & 3] += p;
        }
      psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) pack(mm);
      if (__any(mnew > mrun)) {
        const float alpha = (mnew == -INFINITY) ? 1.f : exp2_hw(mrun - mnew);
        lrun *= alpha;
        // O scaled in place in the accumulation registers (a copy through the
        // vector registers would make the compiler keep O there, at 128
        // registers and two copies per tile).  The last MFMA writing O was
        // issued a whole tile of work earlier; the nops cover the read-after-
        // MFMA, read -> VALU and write -> MFMA source wait states all the same.
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float t;
            asm volatile(
                "v_accvgpr_read_b32 %1, %0\n\t"
                "s_nop 1\n\t"
                "v_mul_f32 %1, %1, %2\n\t"
                "v_accvgpr_write_b32 %0, %1\n\t"
                "s_nop 3"
                : "+a"(o[db][r]), "=&v"(t)
                : "v"(alpha));
          }
      }
    }
    lrun += psum;
    mrun = mnew;
    bf16x8_t vfr[2][8];
    auto ldv = [&](int mm, bf16x8_t (&f)[8]) {
      const bf16_t* vp = vs + vofs[mm];
#pragma unroll
      for (int db = 0; db < 8; ++db) f[db] = as_bf16x8(ldv4(vp + db * 32 * PK));
    };
    ldv(0, vfr[0]);
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      if (mm + 1 < 4) ldv(mm + 1, vfr[(mm + 1) & 1]);
      const bf16x8_t pf = as_bf16x8(u32x4_t{pw[mm][0], pw[mm][1], pw[mm][2], pw[mm][3]});
#pragma unroll
      for (int db = 0; db < 8; ++db) o[db] = mfma32(vfr[mm & 1][db], pf, o[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // keys kv_end .. of the last tile hold arbitrary bits: clear V^T there
  auto mask_tail = [&]() {
    const int kt = ntiles - 1;
    bf16_t* vs = vring + (kt & 1) * A2_KST;
    const int lim = kv_end - kt * PK;
    for (int idx = tid; idx < PD2 * 8; idx += 64 * NW) {
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
  // prologue: K of tiles 0 and 1, V^T of tile 0; scores of tile 0
  issue_k(0);
  if (ntiles > 1) issue_k(1);
  issue_v(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  sync();
  scores(0, sa);
  // step kt: K of tile kt + 1 and V^T of tile kt are in LDS; K of tile kt + 2
  // and V^T of tile kt + 1 go into the stages that tiles kt and kt - 1 used
  // (every wave is past them at the barrier)
  // (par = kt & 1, a constant in each unrolled half, so stage offsets are immediates)
  auto step = [&](int kt, int par, f32x16_t (&cur)[2], f32x16_t (&nxt)[2]) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    sync();
    if (kt + 2 < ntiles) issue_k(kt + 2);
    if (kt + 1 < ntiles) issue_v(kt + 1);
    if (kt == ntiles - 1 && ragged) {
      mask_tail();
      __syncthreads();
    }
    // no branches around these (a branch would make O a merged value, which
    // the compiler keeps in vector registers): past the last tile the scores
    // read a stale stage and go unused; a tile past the wave's last query is
    // masked out whole, so its probabilities are 0
    mask_diag(kt, cur);
    float psum;
    scores_softmax(par ^ 1, nxt, cur, psum);
    rescale_pv(par, cur, psum);
  };
  for (int kt = 0; kt < ntiles; kt += 2) {
    step(kt, 0, sa, sb);
    if (kt + 1 >= ntiles) break;
    step(kt + 1, 1, sb, sa);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load may still target LDS at exit
  if (qvalid) {
    const float ltot = x32_sum(lrun);
    const float inv = 1.0f / ltot;
    bf16_t* O = (bf16_t*)a.out + (size_t)(b * a.S_call + m) * a.ldo + j * PD2;
#pragma unroll
    for (int db = 0; db < 8; ++db)
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
// One workgroup of DW waves (d = 128; DW / 2 at d = 256) per (split, KV head,
// sequence); wave w takes the rounds w, w + DW, ... of the split (64 keys at
// d = 128, 32 at d = 256), so the waves stream neighbouring cache lines
// together.  Query columns c < ncol are (token t = c / G, head kvh*G + c % G).
// A round loads its K rows and its V^T columns at once (32 KB per wave in
// flight), then computes S^T blocks of 16 keys whose rows are ordered so
// that, for PV step kk, lane group g holds the probabilities of keys
// 32kk + 8g + 0..7, matching a contiguous 16-byte read of V^T.  The waves'
// (max, sum, O) are merged in LDS by a fixed tree (w + 4 into w, then w + 2,
// then w + 1).  A single split writes the output; several splits write fp32
// partials for attn_combine.
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

int decode_sk_slots(int Hkv, int cu) {
  const int n = cu / (Hkv > 0 ? Hkv : 1);
  return n > 1 ? n : 1;
}

// about one piece per CU: cu / Hkv pieces per KV head
StreamKPlan decode_plan_sk(int total, int Hkv, int cu) {
  StreamKPlan p{};
  p.slots = decode_sk_slots(Hkv, cu);
  int chunk = (total + p.slots - 1) / p.slots;
  chunk = (chunk + 63) / 64 * 64;
  p.chunk = chunk < 64 ? 64 : chunk;
  p.n_wg = (total + p.chunk - 1) / p.chunk;
  return p;
}

int decode_max_splits(int B, int Hkv, int S_max, int cu) {
  const int groups = B * Hkv > 0 ? B * Hkv : 1;
  const int want = (cu + groups - 1) / groups;
  const int cap = (S_max + 63) / 64;
  return want < 1 ? 1 : (want < cap ? want : cap);
}

// d = 128 takes rounds of 64 keys, d = 256 rounds of 32 keys (the same
// registers per round: K rows and V^T columns of a round in flight at once).
template <int D>
constexpr int decode_waves() { return D == 128 ? DW : DW / 2; }

// Keys [k_begin, min(k_end, kv_len)) of sequence b for KV head kvh: the
// workgroup's waves take the rounds in turn and merge their (max, sum, O) in
// LDS; wave 0 then writes the output (nslot == 1) or the fp32 partial in slot
// `slot` of nslot per row.  Every wave of the workgroup calls this together.
template <int D>
DEV void decode_range(const AttnArgs& a, float* mrg, int b, int kvh, int k_begin, int k_end_cap, int slot, int nslot) {
  constexpr int NWV = decode_waves<D>();    // waves: four at d = 256, each with a whole SIMD's registers
  constexpr int RK = D == 128 ? 64 : 32;     // keys per round
  constexpr int NSB = RK / 16;               // S^T blocks of 16 keys
  constexpr int NKK = RK / 32;               // PV steps of 32 keys
  constexpr int NQ = D / 32;                 // 32-deep q fragments
  constexpr int NO = D / 16;                 // O blocks of 16 rows
  constexpr int NCH = NQ > 4 ? 2 : 1;        // independent score chains per block
  const int G = a.Hq / a.Hkv;
  const int ncol = G * a.S_call;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const bool cvalid = c < ncol;
  const int tq = cvalid ? c / G : 0, jq = kvh * G + (cvalid ? c % G : 0);
  const int pos0 = a.pos_dev ? min(max(a.pos_dev[b], 0), a.pos0) : a.pos0;   // this sequence's first new position
  const int kv_len = pos0 + a.S_call;              // keys [0, kv_len) exist
  const int lim = pos0 + tq + 1;                   // visible to this column
  const int k_end = min(k_end_cap, kv_len);

  const bf16_t* Q = (const bf16_t*)a.q + (size_t)(b * a.S_call + tq) * a.ldq + jq * D;
  bf16x8_t qf[NQ];
  const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int ds = 0; ds < NQ; ++ds) qf[ds] = as_bf16x8(cvalid ? ldv4(Q + ds * 32 + g * 8) : zero);

  const bool paged = a.pages.table != nullptr;
  const bf16_t* Kg = (const bf16_t*)a.kcache + (paged ? 0 : ((size_t)(b * a.Hkv + kvh) * a.S_max) * D);
  const bf16_t* Vg = (const bf16_t*)a.vcache + (paged ? 0 : ((size_t)(b * a.Hkv + kvh) * D) * a.S_max);
  const int vstride = kv_vstride(a.pages, a.S_max);
  const float sc = LOG2E / sqrtf((float)D);

  f32x4_t o[NO];
#pragma unroll
  for (int db = 0; db < NO; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;

  // rounds start at multiples of RK (k_begin is a multiple of 64), so a round
  // lies in one page of a paged cache; its page number is read one round ahead
  int pg = (paged && k_begin + wid * RK < k_end) ? kv_page(a.pages, b, k_begin + wid * RK) : 0;
  for (int k0 = k_begin + wid * RK; k0 < k_end; k0 += NWV * RK) {
    const int pg_next = (paged && k0 + NWV * RK < k_end) ? kv_page(a.pages, b, k0 + NWV * RK) : 0;
    const int in_pg = k0 & (KV_PAGE - 1);
    const bf16_t* Kround = paged ? Kg + (((size_t)pg * a.Hkv + kvh) * KV_PAGE + in_pg) * D : Kg + (size_t)k0 * D;
    const bf16_t* Vround = paged ? Vg + ((size_t)pg * a.Hkv + kvh) * D * KV_PAGE + in_pg : Vg + k0;
    pg = pg_next;
    // loads of the whole round first: K rows (S^T operand) and V^T (PV operand).
    // Keys past k_end stay inside the slot or page (S_max % 64 == 0) and are masked.
    u32x4_t kf[NSB][NQ], vf[NKK][NO];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      const int key = 32 * (sb >> 1) + (c >> 2) * 8 + (sb & 1) * 4 + (c & 3);   // within the round
      const bf16_t* kr = Kround + (size_t)key * D + g * 8;
#pragma unroll
      for (int ds = 0; ds < NQ; ++ds) kf[sb][ds] = ldv4(kr + ds * 32);
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int db = 0; db < NO; ++db) vf[kk][db] = ldv4(Vround + (size_t)(db * 16 + c) * vstride + 32 * kk + 8 * g);

    f32x4_t st[NSB];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      f32x4_t part[NCH];
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        part[ch] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = ch * NQ / NCH; ds < (ch + 1) * NQ / NCH; ++ds)
          part[ch] = mfma16(as_bf16x8(kf[sb][ds]), qf[ds], part[ch]);
      }
      st[sb] = part[0];
#pragma unroll
      for (int ch = 1; ch < NCH; ++ch) st[sb] += part[ch];
    }
    // st[sb][i]: column c, key k0 + 32*(sb/2) + 8g + 4*(sb%2) + i
    float tmax = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
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
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = (mnew == -INFINITY) ? 0.f : exp2_hw(st[sb][i] - mnew);
        st[sb][i] = p;
        psum += p;
      }
    lrun = lrun * alpha + psum;
    mrun = mnew;
#pragma unroll
    for (int db = 0; db < NO; ++db) o[db] *= alpha;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
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
      for (int db = 0; db < NO; ++db) {
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

  // merge waves: step h = NWV / 2, ..., 1: waves [h, 2h) hand their state to w - h
  for (int h = NWV / 2; h >= 1; h >>= 1) {
    if (wid >= h && wid < 2 * h) {
      float* slot = mrg + ((size_t)(wid - h) * 16 + c) * (D + 2);
#pragma unroll
      for (int db = 0; db < NO; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) slot[db * 16 + g * 4 + i] = o[db][i];
      if (g == 0) { slot[D] = mrun; slot[D + 1] = ltot; }
    }
    __syncthreads();
    if (wid < h) {
      const float* slot = mrg + ((size_t)wid * 16 + c) * (D + 2);
      const float m2 = slot[D], l2 = slot[D + 1];
      const float M = fmaxf(mrun, m2);
      const float a1 = (mrun == -INFINITY) ? 0.f : exp2_hw(mrun - M);
      const float a2 = (m2 == -INFINITY) ? 0.f : exp2_hw(m2 - M);
#pragma unroll
      for (int db = 0; db < NO; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[db][i] = o[db][i] * a1 + slot[db * 16 + g * 4 + i] * a2;
      ltot = ltot * a1 + l2 * a2;
      mrun = M;
    }
    __syncthreads();
  }
  if (wid != 0 || !cvalid) return;
  if (nslot == 1) {
    const float inv = 1.f / ltot;
    bf16_t* O = (bf16_t*)a.out + (size_t)(b * a.S_call + tq) * a.ldo + jq * D;
#pragma unroll
    for (int db = 0; db < NO; ++db) {
      const uint32_t w0 = pack_bf16x2(o[db][0] * inv, o[db][1] * inv);
      const uint32_t w1 = pack_bf16x2(o[db][2] * inv, o[db][3] * inv);
      *(u32x2_t*)(O + db * 16 + g * 4) = u32x2_t{w0, w1};
    }
    return;
  }
  float* P = a.part + ((((size_t)(b * a.S_call + tq) * a.Hq + jq) * nslot) + slot) * (D + 2);
#pragma unroll
  for (int db = 0; db < NO; ++db)
    *(float4*)(P + db * 16 + g * 4) = make_float4(o[db][0], o[db][1], o[db][2], o[db][3]);
  if (g == 0) { P[D] = mrun; P[D + 1] = ltot; }
}

// One workgroup of DW waves (d = 128; DW / 2 at d = 256) per (split, KV head,
// sequence): split s covers keys [s split_len, (s + 1) split_len).
template <int D>
__global__ __launch_bounds__(64 * decode_waves<D>()) void attn_decode_mfma(AttnArgs a) {
  extern __shared__ float mrg[];             // [NWV / 2][16][D + 2]: o, max, sum per column
  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  decode_range<D>(a, mrg, b, kvh, s * a.split_len, s * a.split_len + a.split_len, s, a.n_split);
}

// Stream-K split of a ragged batch: the sequences' keys, each padded to a
// multiple of 64, are laid end to end (sequence b at [pref[b], pref[b + 1]))
// and cut into pieces of `chunk` keys (a multiple of 64), one workgroup per
// (piece, KV head), so the work per workgroup is the same whatever the
// lengths.  A piece that spans several sequences yields one partial per
// sequence; sequence b's pieces are pref[b] / chunk .. (pref[b + 1] - 1) /
// chunk, its partial slots 0, 1, ... in that order (a.n_split slots per row).
template <int D>
__global__ __launch_bounds__(64 * decode_waves<D>()) void attn_decode_sk(AttnArgs a, const int32_t* __restrict__ pref,
                                                                         int chunk) {
  extern __shared__ float mrg[];
  const int p = blockIdx.x, kvh = blockIdx.y;
  const int rs = p * chunk, re = min(rs + chunk, pref[a.B]);
  int b = 0;
  while (b < a.B - 1 && pref[b + 1] <= rs) ++b;
  for (; b < a.B && pref[b] < re; ++b) {
    const int base = pref[b];
    decode_range<D>(a, mrg, b, kvh, max(rs, base) - base, min(re, pref[b + 1]) - base, p - base / chunk, a.n_split);
  }
}

template <int D>
constexpr size_t decode_lds() { return (size_t)(decode_waves<D>() / 2) * 16 * (D + 2) * sizeof(float); }

// out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M) over the ns partials of
// one (token, head) row (stored a.n_split apart); thread t takes the
// dimensions t, t + 128, ...
template <typename T>
DEV void combine_row(const AttnArgs& a, int row, int ns) {
  const float* P = a.part + (size_t)row * a.n_split * (a.d + 2);
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, P[s * (a.d + 2) + a.d]);
  float L = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float ms = P[s * (a.d + 2) + a.d];
    L += P[s * (a.d + 2) + a.d + 1] * ((ms == -INFINITY) ? 0.f : exp2_hw(ms - M));
  }
  const int tok = row / a.Hq, j = row % a.Hq;
  for (int dd = threadIdx.x; dd < a.d; dd += 128) {
    float acc = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float ms = P[s * (a.d + 2) + a.d];
      acc += P[s * (a.d + 2) + dd] * ((ms == -INFINITY) ? 0.f : exp2_hw(ms - M));
    }
    st1((T*)a.out + (size_t)tok * a.ldo + j * a.d + dd, acc / L);
  }
}

template <typename T>
__global__ __launch_bounds__(128) void attn_combine(AttnArgs a) {
  combine_row<T>(a, blockIdx.x, a.n_split);     // row (b * S_call + t) * Hq + j
}

// rows of sequence b: its pieces of the stream-K split
template <typename T>
__global__ __launch_bounds__(128) void attn_combine_sk(AttnArgs a, const int32_t* __restrict__ pref, int chunk) {
  const int row = blockIdx.x, b = row / (a.S_call * a.Hq);
  combine_row<T>(a, row, (pref[b + 1] - 1) / chunk - pref[b] / chunk + 1);
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
  const float* K = (const float*)a.kcache;
  const float* V = (const float*)a.vcache;
  const int vstride = kv_vstride(a.pages, a.S_max);
  float qr[D], o[D];
  const float sc = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int i = 0; i < D; ++i) { qr[i] = q[i]; o[i] = 0.f; }
  float m = -INFINITY, l = 0.f;
  const int last = (a.pos_dev ? min(max(a.pos_dev[b], 0), a.pos0) : a.pos0) + t;
  for (int key = 0; key <= last; ++key) {
    const float* Kr = K + kv_k_off(a.pages, a.Hkv, a.S_max, D, b, kvh, key);
    const float* Vc = V + kv_v_off(a.pages, a.Hkv, a.S_max, D, b, kvh, key);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) s += qr[i] * Kr[i];
    s *= sc;
    const float mn = fmaxf(m, s);
    const float al = expf(m - mn), p = expf(s - mn);
    l = l * al + p;
#pragma unroll
    for (int i = 0; i < D; ++i) o[i] = o[i] * al + p * Vc[(size_t)i * vstride];
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
  if (a.Hq % a.Hkv || a.S_max % 64) return hipErrorInvalidValue;
  // a paged cache keeps the page numbers of the workgroup's tiles in LDS past the ring
  const long tiles = ((long)a.pos0 + a.S_call + PK - 1) / PK;
  const size_t pgl = a.pages.table ? (size_t)tiles * sizeof(int) : 0;
  if (a.d == PD2) {
    if (!(G == 1 || G == 2 || G == 4) || A2_LDS + pgl > AQ_LDS_MAX) return hipErrorInvalidValue;
    static bool attr2 = false;
    if (!attr2) {
      hipError_t e = hipFuncSetAttribute((const void*)attn_prefill_d256, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         AQ_LDS_MAX);
      if (e != hipSuccess) return e;
      attr2 = true;
    }
    const int qpw = 32 * (A2_NW / G);
    if ((a.S_call + qpw - 1) / qpw > 65535) return hipErrorInvalidValue;
    dim3 grid(a.Hkv, a.B, (a.S_call + qpw - 1) / qpw);
    attn_prefill_d256<<<grid, 64 * A2_NW, A2_LDS + pgl, s>>>(a);
    return hipGetLastError();
  }
  if (a.d != PD || !(G == 1 || G == 2 || G == 4 || G == 8)) return hipErrorInvalidValue;
  const size_t lds = AQ_LDS + pgl;
  if (lds > AQ_LDS_MAX) return hipErrorInvalidValue;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_prefill_dma, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       AQ_LDS_MAX);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int qpw = 32 * (AQ_NW / G);   // queries per workgroup
  if ((a.S_call + qpw - 1) / qpw > 65535) return hipErrorInvalidValue;
  dim3 grid(a.Hkv, a.B, (a.S_call + qpw - 1) / qpw);
  attn_prefill_dma<<<grid, 64 * AQ_NW, lds, s>>>(a);
  return hipGetLastError();
}

hipError_t attn_decode(const AttnArgs& a, hipStream_t s) {
  if (a.S_call <= 0 || a.B <= 0) return hipSuccess;
  if (a.dt == DT_F32) return launch_f32(a, s);
  const int G = a.Hq / a.Hkv;
  if ((a.d != PD && a.d != PD2) || a.Hq % a.Hkv || G * a.S_call > 16 || a.S_max % 64 || a.split_len % 64)
    return hipErrorInvalidValue;
  const int kv_len = a.pos0 + a.S_call;
  if ((long)a.n_split * a.split_len < kv_len) return hipErrorInvalidValue;
  dim3 grid(a.n_split, a.Hkv, a.B);
  if (a.d == 128) {
    attn_decode_mfma<128><<<grid, 64 * decode_waves<128>(), decode_lds<128>(), s>>>(a);
  } else {
    static bool attr = false;
    if (!attr) {
      hipError_t e = hipFuncSetAttribute((const void*)attn_decode_mfma<256>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)decode_lds<256>());
      if (e != hipSuccess) return e;
      attr = true;
    }
    attn_decode_mfma<256><<<grid, 64 * decode_waves<256>(), decode_lds<256>(), s>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  attn_combine<bf16_t><<<a.B * a.S_call * a.Hq, 128, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t attn_decode_sk(const AttnArgs& a0, const int32_t* pref, const StreamKPlan& p, hipStream_t s) {
  const int G = a0.Hkv > 0 ? a0.Hq / a0.Hkv : 0;
  if (a0.dt != DT_BF16 || (a0.d != PD && a0.d != PD2) || !a0.pos_dev || !pref || a0.Hkv <= 0 || a0.Hq % a0.Hkv ||
      G * a0.S_call > 16 || a0.S_max % 64 || p.chunk % 64 || p.n_wg < 1 || p.slots < p.n_wg)
    return hipErrorInvalidValue;
  if (a0.S_call <= 0 || a0.B <= 0) return hipSuccess;
  AttnArgs a = a0;
  a.n_split = p.slots;                 // partial slots per row
  dim3 grid(p.n_wg, a.Hkv);
  if (a.d == 128) {
    attn_decode_sk<128><<<grid, 64 * decode_waves<128>(), decode_lds<128>(), s>>>(a, pref, p.chunk);
  } else {
    static bool attr = false;
    if (!attr) {
      hipError_t e = hipFuncSetAttribute((const void*)attn_decode_sk<256>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)decode_lds<256>());
      if (e != hipSuccess) return e;
      attr = true;
    }
    attn_decode_sk<256><<<grid, 64 * decode_waves<256>(), decode_lds<256>(), s>>>(a, pref, p.chunk);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  attn_combine_sk<bf16_t><<<a.B * a.S_call * a.Hq, 128, 0, s>>>(a, pref, p.chunk);
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
                                                        int S_max, int pos, KvPages pages) {
  const int n = B * Hkv * d;
  const int vstride = kv_vstride(pages, S_max);
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    const int b = i / (Hkv * d), r = i - b * Hkv * d, hk = r / d, dd = r - hk * d;
    const T* row = qkv + (size_t)b * ld + q_cols;
    kc[kv_k_off(pages, Hkv, S_max, d, b, hk, pos) + dd] = row[hk * d + dd];
    vc[kv_v_off(pages, Hkv, S_max, d, b, hk, pos) + (size_t)dd * vstride] = row[Hkv * d + hk * d + dd];
  }
}

hipError_t kv_append(int dt, const void* qkv, long ld, int q_cols, int B, int Hkv, int d, void* kcache,
                     void* vcache, int S_max, int pos, KvPages pages, hipStream_t s) {
  const int n = B * Hkv * d;
  if (n <= 0) return hipSuccess;
  const int grid = (n + 255) / 256;
  if (dt == DT_BF16)
    kv_append_kernel<bf16_t><<<grid, 256, 0, s>>>((const bf16_t*)qkv, ld, q_cols, B, Hkv, d, (bf16_t*)kcache,
                                                  (bf16_t*)vcache, S_max, pos, pages);
  else
    kv_append_kernel<float><<<grid, 256, 0, s>>>((const float*)qkv, ld, q_cols, B, Hkv, d, (float*)kcache,
                                                 (float*)vcache, S_max, pos, pages);
  return hipGetLastError();
}

// One workgroup per (64-position block, KV head, sequence): K rows go
// straight to the cache; V goes through LDS so that V^T is written as runs of
// consecutive positions.  Only positions pos0 .. pos0 + S - 1 are written (a
// continued chunk shares its first block with earlier positions).  With
// per-sequence start positions (pos_dev, clamped to [0, pos0]) S must be 1.
template <typename T>
__global__ __launch_bounds__(256) void kv_scatter_kernel(const T* __restrict__ qkv, long ld, int q_cols, int S,
                                                         int pos0, const int* __restrict__ pos_dev, int Hkv, int d,
                                                         T* __restrict__ kc, T* __restrict__ vc, int S_max,
                                                         KvPages pages) {
  extern __shared__ __align__(16) unsigned char kvs_raw[];
  T* vl = reinterpret_cast<T*>(kvs_raw);        // [64][d + 1]
  const int dp = d + 1;
  const int hk = blockIdx.y, b = blockIdx.z;
  const int ps = pos_dev ? min(max(pos_dev[b], 0), pos0) : pos0;   // this sequence's first position
  const int p0 = (ps & ~(KV_PAGE - 1)) + KV_PAGE * blockIdx.x;
  const int lo = max(p0, ps), hi = min(p0 + KV_PAGE, ps + S);
  for (int idx = threadIdx.x; idx < KV_PAGE * d; idx += 256) {
    const int r = idx / d, dd = idx - r * d;
    const int pos = p0 + r;
    if (pos >= lo && pos < hi) {
      const T* row = qkv + (size_t)(b * S + pos - ps) * ld + q_cols;
      kc[kv_k_off(pages, Hkv, S_max, d, b, hk, pos) + dd] = row[hk * d + dd];
      vl[r * dp + dd] = row[Hkv * d + hk * d + dd];
    }
  }
  __syncthreads();
  const int vstride = kv_vstride(pages, S_max);
  for (int idx = threadIdx.x; idx < KV_PAGE * d; idx += 256) {
    const int dd = idx / KV_PAGE, r = idx - dd * KV_PAGE;
    const int pos = p0 + r;
    if (pos >= lo && pos < hi) vc[kv_v_off(pages, Hkv, S_max, d, b, hk, pos) + (size_t)dd * vstride] = vl[r * dp + dd];
  }
}

hipError_t kv_scatter(int dt, const void* qkv, long ld, int q_cols, int B, int S, int pos0, const int* pos_dev,
                      int Hkv, int d, void* kcache, void* vcache, int S_max, KvPages pages, hipStream_t s) {
  if (B <= 0 || S <= 0) return hipSuccess;
  if (pos_dev && S != 1) return hipErrorInvalidValue;
  const int blocks = (pos0 + S + KV_PAGE - 1) / KV_PAGE - pos0 / KV_PAGE;
  const dim3 grid(blocks, Hkv, B);
  const size_t es = dt == DT_BF16 ? 2 : 4;
  const size_t lds = (size_t)KV_PAGE * (d + 1) * es;
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  if (dt == DT_BF16)
    kv_scatter_kernel<bf16_t><<<grid, 256, lds, s>>>((const bf16_t*)qkv, ld, q_cols, S, pos0, pos_dev, Hkv, d,
                                                     (bf16_t*)kcache, (bf16_t*)vcache, S_max, pages);
  else
    kv_scatter_kernel<float><<<grid, 256, lds, s>>>((const float*)qkv, ld, q_cols, S, pos0, pos_dev, Hkv, d, (float*)kcache,
                                                    (float*)vcache, S_max, pages);
  return hipGetLastError();
}

}  // namespace lk
