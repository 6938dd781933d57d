// Dense contractions of the looped decoder: C[M, N] = A[M, K] . B[N, K]^T.
//
// * gemm_w16:    bf16, M > 64, K % 128 == 0 (every model shape).  256x256
//                workgroup tile, 4 waves of 128x128 (v_mfma_f32_16x16x32_bf16),
//                64-deep k steps of whole-line global -> LDS DMA into two
//                stages, persistent workgroups, XCD-aware tile order.  fp32
//                accumulation.
// * gemm_dma:    bf16, M > 64, other K % 32 == 0.  The same tile with 8 waves of
//                128x64 and 32-deep steps through five LDS stages.
// * gemm_skinny: bf16, M <= 64 (decode): streams B (the weights) once for up to
//                64 token rows; 128-row tiles whose 4 waves split the rows and share the
//                token operand through LDS; K split, when the tiles cannot fill
//                the device, over workgroups (partials summed in index order
//                by a second kernel).
// * gemm_f32:    fp32 configuration: LDS-tiled FMA kernel.
// All share one epilogue: plain bf16/fp32 store, fp32 logits, the QKV split
// that writes K and V into a per-(layer, pass) cache slot, or SwiGLU.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lk {

// ------------------------------------------------------------------ epilogue
// PG: the cache may be paged.  The 256-row tile kernels take contiguous caches
// only (page addressing there costs the k loop registers); the host stores
// their QKV rows plainly and scatters K / V into the pages (kv_scatter).
template <typename T, bool PG>
DEV void epi_qkv(const GemmArgs& a, int row, int col, float v) {
  if (col < a.q_cols) {
    st1((T*)a.C + (size_t)row * a.ldc + col, v);
    return;
  }
  int cc = col - a.q_cols;
  const int kvn = a.n_kv * a.head_dim;
  const int b = row / a.S_call;
  const int pos = (a.pos_dev ? min(max(a.pos_dev[b], 0), a.pos0) : a.pos0) + row % a.S_call;
  if (cc < kvn) {
    const int hk = cc / a.head_dim, dd = cc % a.head_dim;
    if (PG) st1((T*)a.kcache + kv_k_off(a.pages, a.n_kv, a.S_max, a.head_dim, b, hk, pos) + dd, v);
    else st1((T*)a.kcache + (((size_t)b * a.n_kv + hk) * a.S_max + pos) * a.head_dim + dd, v);
  } else {
    cc -= kvn;
    const int hk = cc / a.head_dim, dd = cc % a.head_dim;
    if (PG)
      st1((T*)a.vcache + kv_v_off(a.pages, a.n_kv, a.S_max, a.head_dim, b, hk, pos) +
              (size_t)dd * kv_vstride(a.pages, a.S_max), v);
    else st1((T*)a.vcache + (((size_t)b * a.n_kv + hk) * a.head_dim + dd) * a.S_max + pos, v);
  }
}

template <typename T, int EPI, bool PG = true>
DEV void epi_one(const GemmArgs& a, int row, int col, float v) {
  if (EPI == EPI_STORE) st1((T*)a.C + (size_t)row * a.ldc + col, v);
  else if (EPI == EPI_F32) ((float*)a.C)[(size_t)row * a.ldc + col] = v;
  else if (EPI == EPI_QKV) epi_qkv<T, PG>(a, row, col, v);
}

// ------------------------------------------------------------------ MFMA tile kernel
// 256x256 workgroup tile; WN_ = 4: 8 waves as 2 (M) x 4 (N), each owning a
// 128x64 sub-tile = 4x2 blocks of v_mfma_f32_32x32x16_bf16 (WN_ = 2: 4 waves
// of 128x128).  Operands move global -> LDS with global_load_lds_dwordx4 (no
// staging registers): BK = 32, five LDS stages, loads issued four tiles
// ahead, LDS fragment reads one k-substep ahead of the MFMAs.  Each
// wave-instruction writes 1 KB of LDS (lane l at +16 l): rows 16 b .. 16 b + 15
// of one operand tile, 64 B each; 16-byte chunk c of row r sits at
// c ^ ((r >> 2) & 3).  SwiGLU: a wave's B rows are JB/2 blocks of gate rows
// then the JB/2 matching up-row blocks, so each wave emits finished output
// columns (128 per workgroup).  Tiles are walked in an XCD-aware order.
constexpr int TBM = 256, TBN = 256;
constexpr int DBK = 32, DST = 5;
constexpr int DSTAGE = (TBM + TBN) * DBK;            // elements per stage (32 KB)
constexpr int GEMM_DMA_LDS = DST * DSTAGE * 2;       // 160 KB

DEV int dswz(int row, int chunk) { return row * DBK + ((chunk ^ ((row >> 2) & 3)) << 3); }

DEV void dma16(const bf16_t* g, bf16_t* l) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)g,
                                   (void __attribute__((address_space(3)))*)l, 16, 0, 0);
}

template <int EPI, int WN_>
__global__ __launch_bounds__(128 * WN_, 1) void gemm_dma_kernel(GemmArgs a) {
  constexpr int JB = 8 / WN_, WCOL = 32 * JB;
  constexpr int NBW = JB;                 // DMA blocks per wave per operand
  extern __shared__ __align__(16) bf16_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / WN_, wn = wid % WN_;
  const int num_m = (a.M + TBM - 1) / TBM;
  const int out_n = (EPI == EPI_SWIGLU) ? 128 : TBN;
  const int num_n = (EPI == EPI_SWIGLU ? a.F : a.N) / out_n;
  const int nblk = num_m * num_n;
  // Consecutive hardware block ids go round-robin over the 8 XCDs: give each
  // XCD a contiguous range of tiles, then walk tiles in groups of 8 row-tiles
  // so neighbouring tiles share A and B panels in that XCD's L2.
  int id = blockIdx.x;
  if (nblk % 8 == 0) id = (id & 7) * (nblk >> 3) + (id >> 3);
  const int GM = 8;
  const int group = GM * num_n;
  const int first_m = (id / group) * GM;
  const int gsz = min(num_m - first_m, GM);
  const int tm = first_m + (id % group) % gsz;
  const int tn = (id % group) / gsz;
  const int m0 = tm * TBM, n0 = tn * out_n;

  // Element offsets fit in 32 bits: the host checks 256*lda and N*ldb < 2^31.
  const bf16_t* A = (const bf16_t*)a.A + (long)m0 * a.lda;
  const bf16_t* B = (const bf16_t*)a.B;
  // wave w issues blocks NBW w .. NBW w + NBW - 1 of A and of B: rows 16 blk + lane / 4
  const int mlast = a.M - 1 - m0;
  int aoff[NBW], boff[NBW], lofs[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int blk = wid * NBW + i;
    const int r = blk * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    aoff[i] = min(r, mlast) * (int)a.lda + c * 8;
    int br;
    if (EPI == EPI_SWIGLU) {
      const int w = r / WCOL, j = (r % WCOL) / 32, cc = r & 31;
      const int oc = n0 + w * (WCOL / 2) + (j % (JB / 2)) * 32 + cc;
      br = (j < JB / 2) ? oc : (a.F + oc);
    } else {
      br = n0 + r;
    }
    boff[i] = br * (int)a.ldb + c * 8;
    lofs[i] = blk * 512;   // elements: 1 KB per block
  }
  const int KT = a.K / DBK;
  // Tiles past the end re-read the last tile into a stage nobody reads
  // again, so every iteration issues the same number of loads and the
  // steady-state loop has no branches (a branch merge makes the compiler
  // drain all outstanding LDS reads).
  auto issue = [&](int kt) {
    bf16_t* st = smem + (kt % DST) * DSTAGE;
    const int k0 = min(kt, KT - 1) * DBK;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      dma16(A + aoff[i] + k0, st + lofs[i]);
      dma16(B + boff[i] + k0, st + TBM * DBK + lofs[i]);
    }
  };
  f32x16_t acc[4][JB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int arow = wm * 128 + (lane & 31);
  const int brow = wn * WCOL + (lane & 31);
  // Software pipeline over k-substeps of 16: the fragments of the next
  // substep are read from LDS while the MFMAs of the current one run.
  bf16x8_t fa[2][4], fb[2][JB];
  auto read_frags = [&](int kt, int ks, bf16x8_t (&xa)[4], bf16x8_t (&xb)[JB]) {
    const bf16_t* as = smem + (kt % DST) * DSTAGE;
    const bf16_t* bs = as + TBM * DBK;
    const int ch = ks * 2 + (lane >> 5);
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) xa[ib] = as_bf16x8(ldv4(as + dswz(arow + ib * 32, ch)));
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) xb[jb] = as_bf16x8(ldv4(bs + dswz(brow + jb * 32, ch)));
  };
  auto mma = [&](const bf16x8_t (&xa)[4], const bf16x8_t (&xb)[JB]) {
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) acc[ib][jb] = mfma32(xa[ib], xb[jb], acc[ib][jb]);
  };
  // Tile j is issued (into stage j % DST) right after the barrier of iteration
  // j - DST + 1.  That barrier guarantees only that every wave has CONSUMED its
  // reads of tile j - DST (their MFMAs ran in the previous iteration), so the
  // issue targets exactly that tile's stage; the stage of the tile being read
  // in this iteration is never written.  Before waiting for tile j at
  // iteration j - 1, the tiles j + 1 .. j + DST - 3 may stay in flight:
  // (DST - 3) * 2 NBW loads (the prologue waits for tile 0 with DST - 2 tiles
  // issued behind it... i.e. (DST - 2) * 2 NBW remaining).
  static_assert(DST == 5, "wait counts below assume five stages");
  auto wait_prologue = [&]() {
    if (NBW == 2) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
  };
  auto wait_tile = [&]() {
    if (NBW == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  };
  // After the barrier every wave's own loads of the waited tile have landed
  // (the wait above), so the whole tile is in LDS.  No memory fence: that
  // would drain the loads still in flight for later tiles.
  auto sync = [&]() {
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };
  for (int t = 0; t < DST - 1; ++t) issue(t);
  wait_prologue();
  sync();
  read_frags(0, 0, fa[0], fb[0]);
  // Interleave the 4 + JB fragment reads of the next substep one-to-one with
  // the MFMAs of the current one, MFMA first (scheduling groups: MFMA, DS read).
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < 4 + JB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * JB - (4 + JB), 0);
  };
  for (int kt = 0; kt + 1 < KT; ++kt) {
    read_frags(kt, 1, fa[1], fb[1]);
    mma(fa[0], fb[0]);
    interleave();
    wait_tile();
    sync();
    issue(kt + DST - 1);      // into the stage of tile kt - 1, consumed before this barrier
    read_frags(kt + 1, 0, fa[0], fb[0]);
    mma(fa[1], fb[1]);
    interleave();
  }
  read_frags(KT - 1, 1, fa[1], fb[1]);
  mma(fa[0], fb[0]);
  mma(fa[1], fb[1]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load may still target LDS at exit

  if (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int jb = 0; jb < JB / 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 128 + ib * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int col = n0 + wn * (WCOL / 2) + jb * 32 + (lane & 31);
          if (row < a.M) {
            const float g = acc[ib][jb][r], u = acc[ib][jb + JB / 2][r];
            st1((bf16_t*)a.C + (size_t)row * a.ldc + col, silu(g) * u);
          }
        }
  } else {
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 128 + ib * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int col = n0 + wn * WCOL + jb * 32 + (lane & 31);
          if (row < a.M) epi_one<bf16_t, EPI, false>(a, row, col, acc[ib][jb][r]);
        }
  }
}

// ------------------------------------------------------------------ MFMA tile kernel, 64-deep
// 256x256 workgroup tile, four waves as 2 (M) x 2 (N), each owning 128x128 =
// 8x8 blocks of v_mfma_f32_16x16x32_bf16 (64 four-register fp32 accumulators,
// 256 per lane).  A k step is 64 deep, so every operand row of a step is one
// whole 128-byte line: a DMA instruction moves 8 rows (1 KB, lane l to
// +16 l), and the row's eight 16-byte chunks sit at c ^ ((row >> 1) & 7): a
// fragment read takes one chunk of 16 consecutive rows per 16 lanes, and with
// 64 four-byte banks two rows span all banks, so the rows of one parity must
// use 8 distinct positions.  Two 64 KB stages; a step is two 32-deep
// substeps of 64 MFMAs with the step's one barrier between them.  Every
// fragment of the second substep is read during the first (two register
// sets, one read after every fourth MFMA), so no wave reads the stage after
// the barrier: the second substep reads the next step's first fragments from
// the other stage, which landed before the barrier, and issues the 16 loads
// of step s + 2 into this stage, one after every fourth MFMA rather than in a
// burst (a burst stalls the wave on a full load queue while its MFMA pipe
// idles).  Scheduling walls after every MFMA fix this order.  The kernel is
// persistent: workgroup b takes tiles b, b + G, ... (G a multiple of 8, at
// most the CU count) as one stream of k steps, so the loads of a tile's
// first steps go out during the previous tile's last steps and the epilogue
// (branch-free buffer stores) runs with them in flight.
// The MFMAs are in-place instructions on the accumulation registers: through
// the builtin the compiler let the registers of the 64 accumulators drift
// between loop iterations and copied them every step.  Against the same tile
// on 32x32x16 MFMAs (sixteen 16-register accumulators, four 16-deep
// substeps) this kernel runs at a higher shader clock under load (1.85
// against 1.69 GHz on the gate/up shape) and was 4-8% faster on every
// Loop-9B projection, with outputs bit for bit equal.
// Against the eight-wave, 32-deep kernel above this halves the L2 requests
// (whole lines) and cuts LDS fragment reads by a third (128x128 per wave).
constexpr int WBK = 64, WST = 2;
constexpr int WSTAGE = (TBM + TBN) * WBK;             // elements per stage (64 KB)
constexpr int GEMM_W16_LDS = WST * WSTAGE * 2;        // 128 KB

DEV int wswz(int row, int chunk) { return row * WBK + ((chunk ^ ((row >> 1) & 7)) << 3); }

// 16 bytes per lane from a buffer (byte offset voff + soff) into LDS at lds + 16 lane.
// Reads past num_records return zeros.
DEV void dma16_buf(__amdgpu_buffer_rsrc_t r, int voff, int soff, bf16_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
DEV __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_w16_kernel(GemmArgs a) {
  constexpr int NB = 8;                    // DMA instructions per wave per operand per step
  extern __shared__ __align__(16) bf16_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid >> 1, wn = wid & 1;
  const int num_m = (a.M + TBM - 1) / TBM;
  const int out_n = (EPI == EPI_SWIGLU) ? 128 : TBN;
  const int num_n = (EPI == EPI_SWIGLU ? a.F : a.N) / out_n;
  const int nblk = num_m * num_n;
  const int G = gridDim.x;
  constexpr int GM = 4;                    // row tiles per group (measured in the whole prefill: 4 over 8 or 16)
  auto tile_mn = [&](int t, int& m0, int& n0) __attribute__((always_inline)) {
    int id = t;
    if (nblk % 8 == 0) id = (id & 7) * (nblk >> 3) + (id >> 3);
    const int group = GM * num_n;
    const int first_m = (id / group) * GM;
    const int gsz = min(num_m - first_m, GM);
    m0 = (first_m + (id % group) % gsz) * TBM;
    n0 = ((id % group) / gsz) * out_n;
  };
  const int KT = a.K / WBK;
  // One load cursor (tile c_t, step c_kt), two steps ahead of the MFMAs.
  // Wave w loads rows 64 w .. 64 w + 63 of both operand tiles: block i is
  // rows 64 w + 8 i + lane / 8.  A lane's whole byte offset of each block
  // sits in a vector register and the scalar offset carries only the k step:
  // with the block's row offset in the scalar operand instead, the kernel ran
  // 25% slower on 24 KB rows (measured).  Rows past M lie past the end of the
  // A view and read zeros.  Offsets fit in 32 bits unsigned (the host checks
  // 256 lda and the B rows against 2^31 elements).
  int c_t = blockIdx.x, c_kt = 0;
  __amdgpu_buffer_rsrc_t Ar;
  const __amdgpu_buffer_rsrc_t Br = buf_rsrc(a.B, 0xFFFFFFF0u);
  const unsigned lda2 = (unsigned)a.lda * 2u, ldb2 = (unsigned)a.ldb * 2u;
  unsigned aoff[NB], boff[NB];
  auto set_ab = [&](int t) __attribute__((always_inline)) {
    int m0, n0;
    tile_mn(t, m0, n0);
    Ar = buf_rsrc((const bf16_t*)a.A + (long)m0 * a.lda, (unsigned)(min(TBM, a.M - m0) * a.lda * 2));
    // B row of tile row r: n0 + r; SwiGLU: rows 128 w' + x are gate rows
    // n0 + 64 w' + x (x < 64), then the up rows of the same outputs
    int brow0;
    if (EPI == EPI_SWIGLU) brow0 = ((wid & 1) ? a.F : 0) + n0 + (wid >> 1) * 64;
    else brow0 = n0 + wid * 64;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int r = 8 * i + (lane >> 3);                          // row within the wave's 64
      const unsigned cs = (unsigned)(((lane & 7) ^ ((r >> 1) & 7)) * 16);
      aoff[i] = (unsigned)(wid * 64 + r) * lda2 + cs;
      boff[i] = (unsigned)(brow0 + r) * ldb2 + cs;
    }
  };
  auto next = [&]() __attribute__((always_inline)) {
    if (++c_kt == KT) {
      if (c_t + G < nblk) {
        c_t += G;
        c_kt = 0;
        set_ab(c_t);
      } else {
        c_kt = KT - 1;      // past the last tile: re-read into the stage nobody reads again
      }
    }
  };
  set_ab(c_t);
  // load L of a step: L < 8 block L of A, else block L - 8 of B
  auto dma = [&](int L, int par) __attribute__((always_inline)) {
    const int i = L % NB;
    if (L < NB) dma16_buf(Ar, (int)aoff[i], c_kt * WBK * 2, smem + par * WSTAGE + (wid * NB + i) * 512);
    else dma16_buf(Br, (int)boff[i], c_kt * WBK * 2, smem + par * WSTAGE + TBM * WBK + (wid * NB + i) * 512);
  };
  f32x4_t acc[8][8];
  const int arow = wm * 128 + (lane & 15);
  const int brow = wn * 128 + (lane & 15);
  bf16x8_t fa[2][8], fb[2][8];
  // the fragment of 16 rows x 32 k: lane l holds row l % 16, k 8 (l / 16) .. + 7 of substep j
  auto read_frags = [&](int par, int j, bf16x8_t (&xa)[8], bf16x8_t (&xb)[8]) __attribute__((always_inline)) {
    const bf16_t* as = smem + par * WSTAGE;
    const bf16_t* bs = as + TBM * WBK;
    const int ch = j * 4 + (lane >> 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xa[i] = as_bf16x8(ldv4(as + wswz(arow + i * 16, ch)));
      xb[i] = as_bf16x8(ldv4(bs + wswz(brow + i * 16, ch)));
    }
  };
  // One substep: 64 MFMAs; after every fourth, one fragment read of the other
  // register set (rd >= 0: substep rd of stage rpar; B blocks first) and, when
  // lpar >= 0, one load into stage lpar.  Scheduling walls keep this order.
  auto substep = [&](const bf16x8_t (&xa)[8], const bf16x8_t (&xb)[8], bool first, int rpar, int rd,
                     bf16x8_t (&ya)[8], bf16x8_t (&yb)[8], int lpar) __attribute__((always_inline)) {
    const bf16_t* as = smem + rpar * WSTAGE;
    const bf16_t* bs = as + TBM * WBK;
    const int ch = rd * 4 + (lane >> 4);
#pragma unroll
    for (int q = 0; q < 64; ++q) {
      const int ib = q >> 3, jb = q & 7;
      if (first)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc[ib][jb]) : "v"(xa[ib]), "v"(xb[jb]));
      else
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[ib][jb]) : "v"(xa[ib]), "v"(xb[jb]));
      if (rd >= 0 && q % 4 == 0) {
        const int f = q / 4;
        if (f < 8) yb[f] = as_bf16x8(ldv4(bs + wswz(brow + f * 16, ch)));
        else ya[f - 8] = as_bf16x8(ldv4(as + wswz(arow + (f - 8) * 16, ch)));
      }
      if (lpar >= 0 && q % 4 == 0) dma(q / 4, lpar);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };
  // step 0 into stage 0; step 1 into stage 1 (lands before step 0's barrier)
#pragma unroll
  for (int L = 0; L < 2 * NB; ++L) dma(L, 0);
  next();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  sync();
#pragma unroll
  for (int L = 0; L < 2 * NB; ++L) dma(L, 1);
  next();
  read_frags(0, 0, fa[0], fb[0]);
  // Step s on stage par: substep 0 reads substep 1's fragments; the barrier
  // (this wave's loads of step s + 1 landed, every read of this stage
  // returned); substep 1 reads the first fragments of step s + 1 (last: of
  // the next tile, after its epilogue instead) and loads step s + 2 here.
  auto step = [&](int par, bool first, bool last) __attribute__((always_inline)) {
    substep(fa[0], fb[0], first, par, 1, fa[1], fb[1], -1);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    sync();
    substep(fa[1], fb[1], false, par ^ 1, last ? -1 : 0, fa[0], fb[0], par);
    next();
  };

  // Epilogue.  acc[ib][jb][r]: row wm*128 + 16 ib + 4 (lane / 16) + r, column
  // wn*128 + 16 jb + lane % 16 (SwiGLU: gate block jb < 4 pairs with up block
  // jb + 4, output column wn*64 + 16 jb + lane % 16).  Plain stores (SwiGLU,
  // bf16 or fp32 output, and QKV tiles wholly in the q columns) go through a
  // buffer view of the tile's rows that ends at row M, so the hardware drops
  // the rows past M and the stores need no branches: a lane's offset is its
  // own column plus a row step that is the same for the whole wave.
  auto epilogue = [&](int m0, int n0) __attribute__((always_inline)) {
    const int lrow = wm * 128 + (lane >> 4) * 4, lcol = lane & 15;
    // QKV tile wholly in the K columns, head_dim 128 (a wave's 128 columns are
    // one KV head) and rows in one sequence: its K-cache rows [pos][d] are a
    // plain row-major block, stored like the q tiles
    int ksq = -1;
    if (EPI == EPI_QKV && n0 >= a.q_cols && n0 + TBN <= a.q_cols + a.n_kv * a.head_dim && a.head_dim == 128 &&
        !a.pos_dev && m0 / a.S_call == (min(m0 + TBM, a.M) - 1) / a.S_call)
      ksq = m0 / a.S_call;
    if (EPI == EPI_SWIGLU || EPI == EPI_STORE || EPI == EPI_F32 || n0 + TBN <= a.q_cols || ksq >= 0) {
      constexpr int ES = EPI == EPI_F32 ? 4 : 2;
      int ldcb = (int)(ksq >= 0 ? a.head_dim : a.ldc) * ES;
      // opaque here, so the 32 row offsets below are formed per tile rather
      // than hoisted out of the tile loop, where they would hold registers
      asm volatile("" : "+s"(ldcb));
      const char* base = (const char*)a.C + (size_t)m0 * ldcb;
      int lb = lrow * ldcb + (n0 + wn * (EPI == EPI_SWIGLU ? 64 : 128) + lcol) * ES;
      if (ksq >= 0) {
        const int hk = (n0 - a.q_cols) / 128 + wn;
        base = (const char*)a.kcache +
               (((size_t)ksq * a.n_kv + hk) * a.S_max + a.pos0 + (m0 - ksq * a.S_call)) * (size_t)ldcb;
        lb = lrow * ldcb + lcol * ES;
      }
      const __amdgpu_buffer_rsrc_t Cr = buf_rsrc(base, (unsigned)(min(TBM, a.M - m0) * ldcb));
#pragma unroll
      for (int ib = 0; ib < 8; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int vo = lb + (ib * 16 + r) * ldcb;
          if (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
              __builtin_amdgcn_raw_buffer_store_b16(f2bf(silu(acc[ib][jb][r]) * acc[ib][jb + 4][r]), Cr,
                                                    vo + jb * 16 * ES, 0, 0);
          } else if (EPI == EPI_F32) {
#pragma unroll
            for (int jb = 0; jb < 8; ++jb)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[ib][jb][r]), Cr, vo + jb * 16 * ES, 0, 0);
          } else {
#pragma unroll
            for (int jb = 0; jb < 8; ++jb)
              __builtin_amdgcn_raw_buffer_store_b16(f2bf(acc[ib][jb][r]), Cr, vo + jb * 16 * ES, 0, 0);
          }
        }
    } else {
      // QKV: a tile wholly in the V columns writes V^T [.., d][S_max]: a lane's
      // four rows of a block are four consecutive positions of one column, so
      // they go out as one 8-byte store (same sequence and 4-aligned positions
      // when S_call and pos0 are multiples of 4); other tiles element by element
      const int kvn = a.n_kv * a.head_dim;
      const bool vtile = EPI == EPI_QKV && n0 >= a.q_cols + kvn && !a.pos_dev && a.S_call % 4 == 0 &&
                         a.pos0 % 4 == 0 && (a.head_dim & 31) == 0;
#pragma unroll
      for (int ib = 0; ib < 8; ++ib)
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) {
          const int row = m0 + lrow + ib * 16;      // rows row .. row + 3
          const int col = n0 + wn * 128 + jb * 16 + lcol;
          if (vtile && row + 3 < a.M) {
            const int cc = col - a.q_cols - kvn;
            const int hk = cc / a.head_dim, dd = cc - hk * a.head_dim;
            const int b = row / a.S_call, pos = a.pos0 + row - b * a.S_call;
            bf16_t* dst = (bf16_t*)a.vcache + (((size_t)b * a.n_kv + hk) * a.head_dim + dd) * a.S_max + pos;
            *(u32x2_t*)dst = u32x2_t{pack_bf16x2(acc[ib][jb][0], acc[ib][jb][1]),
                                     pack_bf16x2(acc[ib][jb][2], acc[ib][jb][3])};
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (row + r < a.M) epi_one<bf16_t, EPI, false>(a, row + r, col, acc[ib][jb][r]);
          }
        }
    }
  };

  for (int t = blockIdx.x; t < nblk; t += G) {
    step(0, true, false);
    for (int kt = 1; kt + 2 < KT; kt += 2) {
      step(1, false, false);
      step(0, false, false);
    }
    step(1, false, true);
    int m0, n0;
    tile_mn(t, m0, n0);
    // the in-place MFMAs are opaque to the compiler's hazard checks: wait out
    // their write latency before the accumulators are read.  The empty
    // statements after the wait redefine every accumulator, so no read of one
    // can be scheduled above the wait.
    asm volatile("s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
#pragma unroll
    for (int ib = 0; ib < 8; ++ib)
#pragma unroll
      for (int jb = 0; jb < 8; ++jb) asm volatile("" : "+a"(acc[ib][jb]));
    epilogue(m0, n0);
    read_frags(0, 0, fa[0], fb[0]);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load may still target LDS at exit
}

// ------------------------------------------------------------------ skinny (M <= 64)
// Decode shape: the weights are streamed once; the <= 64 token rows (one or two
// blocks of 32) are the MFMA's other operand (gemm_skinny_rs_kernel below).
// ksplit == 1: the workgroup applies the epilogue.  ksplit > 1: it stores its
// fp32 partial tile and gemm_skinny_reduce (the next kernel on the stream, so
// the kernel boundary orders the partials) adds the ksplit partials in index
// order and applies the epilogue: results do not depend on scheduling.
constexpr int SK_THREADS = 256;

// Tiles of 128 weight rows (SwiGLU: 64 output columns).  K is split in powers
// of two (at most 16) while the grid has fewer than two workgroups per CU and
// each workgroup keeps a multiple of four 64-wide k steps, at least sixteen, or
// at least eight while the grid is still under one workgroup per CU (the
// streaming rate of a workgroup falls with fewer steps: the first loads'
// latency is paid once per workgroup).
SkinnyPlan skinny_plan(int epi, int M, int N, int K, int F, int cu) {
  SkinnyPlan p{};
  auto tiles_of = [&](int rb) {
    const int rows = 32 * rb;
    return (epi == EPI_SWIGLU) ? (F + rows / 2 - 1) / (rows / 2) : (N + rows - 1) / rows;
  };
  p.tb = M > 32 ? 2 : 1;
  p.rb = 4;
  p.tiles = tiles_of(p.rb);
  p.ksplit = 1;
  for (;;) {
    const int ks2 = 2 * p.ksplit;
    if (p.ksplit >= 16 || (long)p.tiles * p.ksplit >= 2L * cu || K % (ks2 * 4 * 64)) break;
    const int steps2 = K / (ks2 * 64);
    if (!(steps2 >= 16 || (steps2 >= 8 && (long)p.tiles * p.ksplit < cu))) break;
    p.ksplit = ks2;
  }
  if (p.ksplit > 1) p.bytes = (size_t)p.tiles * p.ksplit * 32 * p.tb * 32 * p.rb * sizeof(float);
  return p;
}

template <int EPI, int RB>
DEV void sk_epilogue(const GemmArgs& a, int tile, int m, int j, float v, float vup) {
  constexpr int R = 32 * RB;
  if (EPI == EPI_SWIGLU) {
    const int col = tile * (R / 2) + j;
    if (col < a.F) st1((bf16_t*)a.C + (size_t)m * a.ldc + col, silu(v) * vup);
  } else {
    const int col = tile * R + j;
    if (col < a.N) epi_one<bf16_t, EPI>(a, m, col, v);
  }
}

// One thread per output (token m, output column): the ksplit partials of its
// tile in index order, then the epilogue.
template <int EPI, int RB, int TB>
__global__ __launch_bounds__(256) void gemm_skinny_reduce(GemmArgs a) {
  constexpr int R = 32 * RB, TOK = 32 * TB;
  constexpr int per_tile = (EPI == EPI_SWIGLU) ? R / 2 : R;
  const int tiles = (EPI == EPI_SWIGLU) ? (a.F + per_tile - 1) / per_tile : (a.N + R - 1) / R;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.M * tiles * per_tile) return;
  const int m = i / (tiles * per_tile), c = i - m * tiles * per_tile;
  const int tile = c / per_tile, j = c - tile * per_tile;
  const int ks = a.ksplit;
  const float* p = a.part + (size_t)tile * ks * TOK * R + m * R + j;
  float v = 0.f, vup = 0.f;
  for (int q = 0; q < ks; ++q) {
    v += p[(size_t)q * TOK * R];
    if (EPI == EPI_SWIGLU) vup += p[(size_t)q * TOK * R + R / 2];
  }
  sk_epilogue<EPI, RB>(a, tile, m, j, v, vup);
}

// ------------------------------------------------------------------ skinny, row split
// Decode shape with the token operand shared: a workgroup owns 128 weight rows
// (SwiGLU: 64 gate and the 64 matching up rows) and a k range; each of its four
// waves owns one 32-row MFMA block (SwiGLU: 16 gate rows, then their 16 up
// rows) over the whole range, so all four read the same token operand.
// Both operands move global -> LDS by DMA in whole 128-byte lines, D steps of
// 64 k ahead: the tokens into a ring shared by the workgroup, the weights into
// a ring private to each wave (one DMA instruction moves 8 rows x 128 B).
// Reading the weights straight into registers would have each load touch 64
// lines (32 rows x two 16-byte pieces) and caps a workgroup near 20 GB/s.
// k order inside a step: lane half h takes k + 32 h .. + 31; MFMA j takes
// 16-byte chunk 4 h + j of both operands.  Rows [n][64 k] in LDS (tokens and
// weights alike): chunk c of row n at slot c ^ ((n >> 1) & 7).
// ksplit > 1: fp32 partial tiles [blockIdx][TOK][128] in the logical column
// order (SwiGLU: gate columns, then up columns), read by gemm_skinny_reduce<.., 4, TB>
// or a YPart consumer; ksplit == 1: the epilogue is applied directly.
template <int EPI, int TB, int D>
__global__ __launch_bounds__(SK_THREADS) void gemm_skinny_rs_kernel(GemmArgs a) {
  constexpr int R = 128, TOK = 32 * TB, NS = D + 1;
  constexpr int TSTAGE = TOK * 64, WSTAGE = 32 * 64;             // elements per stage
  constexpr int RING = NS * (TSTAGE + 4 * WSTAGE) * 2, STAGE_OUT = TOK * (R + 1) * 4;
  __shared__ __align__(16) char lds[RING > STAGE_OUT ? RING : STAGE_OUT];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  bf16_t* As = (bf16_t*)lds;                                      // [NS][TOK][64]
  bf16_t* Ws = As + NS * TSTAGE + wid * NS * WSTAGE;              // this wave's [NS][32][64]
  const int ks = a.ksplit;
  const int tile = blockIdx.x / ks, kpart = blockIdx.x - tile * ks;
  const int r = lane & 31, h = lane >> 5;
  const int Kw = a.K / ks, kb = kpart * Kw;
  const int nsteps = Kw / 64;
  // weight DMA i: rows 8 i .. 8 i + 7 of the wave's block; lane l writes slot
  // l % 8 of row 8 i + l / 8, so it fetches the chunk the swizzle puts there
  const bf16_t* Bg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ ((rl >> 1) & 7);
    int n;
    if (EPI == EPI_SWIGLU) {
      const int j = tile * 64 + wid * 16 + (rl & 15);               // output column
      n = j < a.F ? (rl < 16 ? j : a.F + j) : 0;
    } else {
      n = tile * R + wid * 32 + rl;
      n = n < a.N ? n : 0;
    }
    Bg[i] = (const bf16_t*)a.B + (size_t)n * a.ldb + kb + c * 8;
  }
  // token DMA: per step TOK rows of 128 B = 4 TB blocks of 8 rows; wave w
  // issues blocks w + 4 i, with the same lane-to-slot rule
  const bf16_t* Ag[TB];
  int Al[TB];
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    const int blk = wid + 4 * i, t = 8 * blk + (lane >> 3);
    const int c = (lane & 7) ^ ((t >> 1) & 7);
    Ag[i] = (const bf16_t*)a.A + (size_t)min(t, a.M - 1) * a.lda + kb + c * 8;
    Al[i] = blk * 512;
  }
  auto dma = [](const bf16_t* g, bf16_t* l) {
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)g,
                                     (void __attribute__((address_space(3)))*)l, 16, 0, 0);
  };
  auto issue = [&](int st) {      // weights and tokens of step st
    // the weight stage refilled here last held step st - D - 1; the wait makes
    // every LDS read this wave has issued (those of that step included) return
    // before the DMA can overwrite it
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    bf16_t* wd = Ws + (st % NS) * WSTAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma(Bg[i] + st * 64, wd + i * 512);
    bf16_t* td = As + (st % NS) * TSTAGE;
#pragma unroll
    for (int i = 0; i < TB; ++i) dma(Ag[i] + st * 64, td + Al[i]);
  };
  f32x16_t acc[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[tb][i] = 0.f;
  auto sync = [&]() {
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };
  auto compute = [&](int st) {
    const bf16_t* ws = Ws + (st % NS) * WSTAGE;
    const bf16_t* src = As + (st % NS) * TSTAGE;
    u32x4_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = ldv4(ws + r * 64 + (((4 * h + j) ^ ((r >> 1) & 7)) << 3));
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int t = tb * 32 + r;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4_t x = ldv4(src + t * 64 + (((4 * h + j) ^ ((t >> 1) & 7)) << 3));
        acc[tb] = mfma32(as_bf16x8(w[j]), as_bf16x8(x), acc[tb]);
      }
    }
  };
  // Group of step st = 4 weight DMAs then TB token DMAs.  Waiting until at
  // most (D - 1 - q) groups are outstanding lands the oldest one; the barrier
  // then makes every wave's token rows of that step visible, and also orders
  // all reads of step st - 1 before the DMA that refills its token stage.
  constexpr int GS = 4 + TB;
  static_assert(GS * (D - 1) <= 63, "vmcnt range");
  auto wait_groups = [&](auto q) {
    constexpr int N = GS * (D - 1 - decltype(q)::value);
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
  };
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d);
  int st = 0;
  for (; st + D < nsteps; st += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      wait_groups(std::integral_constant<int, 0>{});
      sync();
      compute(st + d);
      issue(st + d + D);          // stages of step st + d - 1, read before the barrier above
    }
  }
  // last D steps: no more loads, the outstanding groups drain one by one
  wait_groups(std::integral_constant<int, 0>{}); sync(); compute(st);
  if constexpr (D > 1) { wait_groups(std::integral_constant<int, 1>{}); sync(); compute(st + 1); }
  if constexpr (D > 2) { wait_groups(std::integral_constant<int, 2>{}); sync(); compute(st + 2); }
  if constexpr (D > 3) { wait_groups(std::integral_constant<int, 3>{}); sync(); compute(st + 3); }
  static_assert(D <= 4, "drain above");

  // accumulators -> LDS in the logical column order, then coalesced output
  sync();                              // every wave is done with both rings
  float* out = (float*)lds;            // [TOK][R + 1]
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int wr = (i >> 2) * 8 + h * 4 + (i & 3);      // row inside the wave's block
      int col;
      if (EPI == EPI_SWIGLU) col = wr < 16 ? wid * 16 + wr : 64 + wid * 16 + (wr - 16);
      else col = wid * 32 + wr;
      out[(tb * 32 + r) * (R + 1) + col] = acc[tb][i];
    }
  __syncthreads();
  const int M = a.M;
  if (ks > 1) {
    float* mine = a.part + (size_t)blockIdx.x * TOK * R;
    for (int e = tid; e < M * R; e += SK_THREADS) mine[e] = out[(e / R) * (R + 1) + e % R];
    return;
  }
  if (EPI == EPI_SWIGLU) {
    for (int e = tid; e < M * 64; e += SK_THREADS) {
      const int t = e / 64, j = e % 64, col = tile * 64 + j;
      if (col < a.F)
        st1((bf16_t*)a.C + (size_t)t * a.ldc + col, silu(out[t * (R + 1) + j]) * out[t * (R + 1) + 64 + j]);
    }
  } else {
    for (int e = tid; e < M * R; e += SK_THREADS) {
      const int t = e / R, j = e % R, col = tile * R + j;
      if (col < a.N) epi_one<bf16_t, EPI>(a, t, col, out[t * (R + 1) + j]);
    }
  }
}

// Four steps in flight (a 100-120 KB ring, one workgroup per CU) while the
// grid has at most one workgroup per CU or each workgroup streams at least 32
// steps; two (60-72 KB, two per CU) otherwise.
template <int EPI, int TB>
static hipError_t launch_skinny_rs(const GemmArgs& a, hipStream_t s) {
  const int tiles = (EPI == EPI_SWIGLU) ? (a.F + 63) / 64 : (a.N + 127) / 128;
  const int steps = a.K / (a.ksplit * 64);
  const int grid = tiles * a.ksplit;
  static int cu = 0;
  if (cu == 0) cu = device_cu_count() > 0 ? device_cu_count() : 256;
  if (steps % 4 == 0 && (grid <= cu || steps >= 32)) gemm_skinny_rs_kernel<EPI, TB, 4><<<grid, SK_THREADS, 0, s>>>(a);
  else if (steps % 2 == 0) gemm_skinny_rs_kernel<EPI, TB, 2><<<grid, SK_THREADS, 0, s>>>(a);
  else gemm_skinny_rs_kernel<EPI, TB, 1><<<grid, SK_THREADS, 0, s>>>(a);
  if (a.ksplit > 1 && !(a.defer_reduce && EPI == EPI_STORE)) {
    const long outs = (long)a.M * tiles * (EPI == EPI_SWIGLU ? 64 : 128);
    gemm_skinny_reduce<EPI, 4, TB><<<(int)((outs + 255) / 256), 256, 0, s>>>(a);
  }
  return hipGetLastError();
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
template <int EPI, int WN_>
static hipError_t launch_dma(const GemmArgs& a, int blocks, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_dma_kernel<EPI, WN_>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, GEMM_DMA_LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  gemm_dma_kernel<EPI, WN_><<<blocks, 128 * WN_, GEMM_DMA_LDS, s>>>(a);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_w16(const GemmArgs& a, int blocks, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_w16_kernel<EPI>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       GEMM_W16_LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  gemm_w16_kernel<EPI><<<blocks, 256, GEMM_W16_LDS, s>>>(a);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 64) {
    if (a.ksplit < 1 || a.K % (a.ksplit * 64)) return hipErrorInvalidValue;
    if (a.ksplit > 1 && !a.part) return hipErrorInvalidValue;
    return a.M > 32 ? launch_skinny_rs<EPI, 2>(a, s) : launch_skinny_rs<EPI, 1>(a, s);
  }
  if (a.K % DBK || (EPI == EPI_QKV && a.pages.table)) return hipErrorInvalidValue;
  if ((long)TBM * a.lda >= (1L << 31) || (long)(EPI == EPI_SWIGLU ? 2 * a.F : a.N) * a.ldb >= (1L << 31) ||
      (long)TBM * a.ldc * 4 >= (1L << 31))
    return hipErrorInvalidValue;
  const int out_n = (EPI == EPI_SWIGLU) ? 128 : TBN;
  const int ncols = (EPI == EPI_SWIGLU) ? a.F : a.N;
  if (ncols % out_n) return hipErrorInvalidValue;
  const int blocks = ((a.M + TBM - 1) / TBM) * (ncols / out_n);
  if (a.K % (2 * WBK) == 0) {
    // persistent: one workgroup per CU (a multiple of 8, for the XCD order)
    const int cu = device_cu_count() & ~7;
    return launch_w16<EPI>(a, (cu > 0 && blocks > cu) ? cu : blocks, s);
  }
  return launch_dma<EPI, 4>(a, blocks, s);
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
