// Projections for larger batches and prefill: a register-blocked MFMA GEMM
// on fp16 activations and weights (v_mfma_f32_16x16x32_f16, fp32
// accumulate), split over K when the output has too few tiles to fill the
// chip.  The small-batch GEMV is in k_gemv.hip.
#include "launch.h"

#include <stdio.h>
#include <string.h>

// ============================================================== MFMA GEMM
// out[m][n] = epi(sum_k A[m][k] W[n][k]) with fp16 A (activations, k
// contiguous) and fp16 W (weights, k contiguous), fp32 accumulation on
// v_mfma_f32_16x16x32_f16.
//
// Workgroup: 4 waves as 2 x 2, each owning a (16 TM) x (16 TN) block of the
// (32 TM) x (32 TN) tile, TM x TN accumulators of 16 x 16.  K advances in
// stages of KS (32, 64 or 128): the next stage's A and W tiles are loaded
// into registers (16-byte loads) while the current stage is multiplied out
// of LDS, then written to the other LDS buffer; one barrier per stage.  In
// the MFMA operand layout lane l holds row l % 16 and the 8 k values
// 8 (l / 16) .. +7 of a 32-wide k slice, for both operands, so A and W
// fragments are plain 16-byte LDS reads of k-contiguous rows.
//
// Column tiles never straddle a segment (each segment has its own
// activation and epilogue).  With split > 1 each tile's stages are divided
// into `split` contiguous ranges whose fp32 partial sums a second kernel adds
// in a fixed order before applying the epilogue, so results do not depend
// on scheduling.
// LDS rows are KS + 16 halves: with a row stride of KS + 8 halves the
// fragment reads and the staging writes still meet bank conflicts on gfx950
// (measured with SQ_LDS_BANK_CONFLICT); + 16 removes them.
constexpr int MM_PAD = 16;

// Epilogue of a workgroup's tile (acc in the MFMA D layout: lane l holds
// rows 4 (l / 16) + e, column l % 16 of each 16 x 16 block).  With one K
// range the segment's epilogue runs here; with several, each range stores
// its fp32 partial sums and k_mm_reduce adds them in range order.  (Adding
// them in the last range to finish needs device-scope release / acquire
// fences, which on gfx950 write back and invalidate the whole L2 of the
// XCD under the running GEMM: measured 2.5 - 5x slower than the extra
// launch.)
template <int TM, int TN>
__device__ __forceinline__ void mm_epilogue(const ProjArgs& a, const Seg& sg, const floatx4 (&acc)[TM][TN],
                                            int ks_id, int n0, int m0, int wm0, int wn0, int lane) {
  const int fr = lane & 15;
  const int er = (lane >> 4) * 4;
  float* P = a.part + (long)ks_id * a.M * a.total_rows;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn0 + 16 * j + fr;
      if (n >= sg.row1) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm0 + 16 * i + er + e;
        if (m >= a.M) continue;
        if (a.split > 1)
          P[(long)m * a.total_rows + n] = acc[i][j][e];
        else
          epi_store(sg, n - sg.row0, m, acc[i][j][e]);
      }
    }
}

// Writes `rows` rows of a tile staged in LDS (NT + 4 floats apart) to the
// output rows mr0 .. mr0 + rows - 1 (or to this K range's partial sums).
template <int NT>
__device__ __forceinline__ void mm_store_rows(const ProjArgs& a, const Seg& sg, const float* smem, int rows,
                                              bool split, float* P, bool f16, int n0, int mr0) {
  constexpr int LDR = NT + 4;
  constexpr int C4 = NT / 4;
  for (int c = threadIdx.x; c < rows * C4; c += blockDim.x) {
    const int r = c / C4, c4 = (c % C4) * 4;
    const int m = mr0 + r, n = n0 + c4;
    if (m >= a.M || n >= sg.row1) continue;
    const floatx4 v = *reinterpret_cast<const floatx4*>(&smem[r * LDR + c4]);
    const bool whole = n + 3 < sg.row1;
    if (split) {
      float* q = P + (long)m * a.total_rows + n;
      if (whole && ((uintptr_t)q & 15) == 0) {
        stf4(q, v);
      } else {
        for (int k = 0; k < 4 && n + k < sg.row1; ++k) q[k] = v[k];
      }
      continue;
    }
    const int nl = n - sg.row0;
    const long o = (long)m * sg.ld_out + nl;
    const bool vec = whole && (f16 ? (((uintptr_t)((half_t*)sg.out + o) & 7) == 0)
                                   : (((uintptr_t)((float*)sg.out + o) & 15) == 0));
    if (!vec) {
      for (int k = 0; k < 4 && n + k < sg.row1; ++k) epi_store(sg, nl + k, m, v[k]);
      continue;
    }
    floatx4 rs = {0.f, 0.f, 0.f, 0.f};
    if (sg.epi == EPI_RESID) {
      if (f16) {
        const half4 h = *reinterpret_cast<const half4*>((const half_t*)sg.out + o);
        rs = floatx4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
      } else {
        rs = ldf4((const float*)sg.out + o);
      }
    }
    floatx4 out;
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = epi_value(sg, nl + k, v[k], rs[k]);
    if (f16) {
      half4 h;
#pragma unroll
      for (int k = 0; k < 4; ++k) h[k] = (half_t)out[k];
      *reinterpret_cast<half4*>((half_t*)sg.out + o) = h;
    } else {
      stf4((float*)sg.out + o, out);
    }
  }
}


// The same through LDS: the tile's sums go to `smem` (RCH rows of NT + 4
// floats at a time; the stage buffers are free once the K loop is done),
// then every thread writes runs of four columns of a row with one 16-byte
// store (fp32) or 8-byte store (fp16), instead of the MFMA layout's single
// floats.  Ragged edges and unaligned outputs take the single-element path.
// A tile larger than the buffers goes out in chunks of RCH rows.  (Every
// accumulator index here is a compile-time constant; the single-float
// epilogue above, unrolled over 32 or more accumulator blocks, is not fully
// unrolled by the compiler, which then keeps the whole accumulator array in
// scratch memory, main loop included.)
template <int TM, int TN, int MT, int NT, int RCH = MT>
__device__ __forceinline__ void mm_epilogue_lds(const ProjArgs& a, const Seg& sg, const floatx4 (&acc)[TM][TN],
                                                int ks_id, int n0, int m0, int wm0, int wn0, int lane,
                                                float* smem) {
  static_assert(RCH % 16 == 0 && MT % RCH == 0, "whole 16-row blocks per chunk");
  constexpr int LDR = NT + 4;
  constexpr int C4 = NT / 4;
  const int fr = lane & 15;
  const int er = (lane >> 4) * 4;
  const bool split = a.split > 1;
  float* P = a.part + (long)ks_id * a.M * a.total_rows;
  const bool f16 = sg.out_f16 != 0;
#pragma unroll
  for (int c0 = 0; c0 < MT; c0 += RCH) {
    __syncthreads();   // every wave is done reading the stage buffers (or the previous chunk)
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int rb = wm0 + 16 * i - c0;   // the block's first row in this chunk (uniform per wave)
      if (RCH < MT && (rb < 0 || rb >= RCH)) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) smem[(rb + er + e) * LDR + wn0 + 16 * j + fr] = acc[i][j][e];
    }
    __syncthreads();
    mm_store_rows<NT>(a, sg, smem, RCH, split, P, f16, n0, m0 + c0);
  }
}
// PIPE = 1 runs the K loop as a three-deep software pipeline (LDS fragment
// reads of the next stage overlap the current stage's MFMAs); it costs
// 2 (TM + TN) KS / 32 fragment registers and pays off on some shapes only.
// PIPE = 2 keeps two stages of global loads in flight (see below); the
// LDS-DMA variant k_mm_dma (K loop 3) is further down.
template <int TM, int TN, int KS, int PIPE>
__global__ __launch_bounds__(256) void k_mm(ProjArgs a) {
  constexpr int MT = 32 * TM, NT = 32 * TN;
  constexpr int CPR = KS / 8;          // 16-byte chunks per row and stage
  constexpr int ACH = MT * CPR / 256;  // 16-byte A chunks per thread and stage
  constexpr int BCH = NT * CPR / 256;  // 16-byte W chunks per thread and stage
  constexpr int LDSR = KS + MM_PAD;    // halves per LDS row
  // stage buffers: A rows 0 .. MT - 1, then the W rows (one array, so the
  // epilogue can reuse it as one block)
  __shared__ __attribute__((aligned(16))) half_t Sm[2][MT + NT][LDSR];

  // XCD-aware order: consecutive work items (same column tile, successive
  // M tiles and K ranges) go to the same XCD, whose L2 then serves the
  // repeated weight and activation reads.
  const int n_tiles = a.tile0[a.nseg];
  const int total = n_tiles * a.m_tiles * a.split;
  const int per_xcd = (total + 7) / 8;
  const int lin = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (lin >= total) return;
  const int ks_id = lin % a.split;
  const int m_tile = (lin / a.split) % a.m_tiles;
  const int n_tile = lin / (a.split * a.m_tiles);
  // segment of this column tile (selects, not a dynamic index into the arguments)
  Seg sg = a.seg[0];
  int t0 = 0;
#pragma unroll
  for (int i = 1; i < MAX_SEGS; ++i)
    if (i < a.nseg && n_tile >= a.tile0[i]) {
      sg = a.seg[i];
      t0 = a.tile0[i];
    }
  const int n0 = sg.row0 + (n_tile - t0) * NT;   // first output column (global)
  const int m0 = m_tile * MT;
  const bool own = sg.W != nullptr;
  const int K = own ? sg.K : a.K;
  const half_t* Wb = own ? sg.W - (long)sg.row0 * K : a.W;  // indexed by global column
  const half_t* A = reinterpret_cast<const half_t*>(sg.act) + sg.act_off;
  const int lda = sg.ld_act;
  const int nst = (K + KS - 1) / KS;
  const int st0 = (int)((long)nst * ks_id / a.split);
  const int st1 = (int)((long)nst * (ks_id + 1) / a.split);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm0 = (wave >> 1) * 16 * TM;
  const int wn0 = (wave & 1) * 16 * TN;
  const int fr = lane & 15;          // fragment row / column
  const int fk = (lane >> 4) * 8;    // fragment k offset inside a 32-wide slice

  floatx4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[ACH], rb[BCH];
  auto load = [&](int stg) {
    const int k0 = stg * KS;
#pragma unroll
    for (int p = 0; p < ACH; ++p) {
      const int c = p * 256 + tid;
      const int r = c / CPR, kc = (c % CPR) * 8;
      const int m = m0 + r;
      ra[p] = (m < a.M && k0 + kc < K) ? ld16(A + (long)m * lda + k0 + kc) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int p = 0; p < BCH; ++p) {
      const int c = p * 256 + tid;
      const int r = c / CPR, kc = (c % CPR) * 8;
      const int n = n0 + r;
      rb[p] = (n < sg.row1 && k0 + kc < K) ? ld16(Wb + (long)n * K + k0 + kc) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int p = 0; p < ACH; ++p) {
      const int c = p * 256 + tid;
      st16(&Sm[buf][c / CPR][(c % CPR) * 8], ra[p]);
    }
#pragma unroll
    for (int p = 0; p < BCH; ++p) {
      const int c = p * 256 + tid;
      st16(&Sm[buf][MT + c / CPR][(c % CPR) * 8], rb[p]);
    }
  };

  if constexpr (PIPE == 2) {
  // Two stages in flight in registers.  The loads read clamped (always
  // valid) addresses and are issued unconditionally in the steady-state
  // loop, so the waitcnt before each LDS write waits for its own stage
  // only; k beyond K is zeroed when written to LDS.  The scheduling
  // barriers keep the loads at the top of each stage (left alone, the
  // scheduler sinks them below the MFMAs and the latency is exposed).
  const int mlast = a.M - 1, nlast = sg.row1 - 1, klast = K - 8;
  u32x4 qa[2][ACH], qb[2][BCH];
  auto load2 = [&](int stg, u32x4* pa, u32x4* pb) {
    const int k0 = stg * KS;
#pragma unroll
    for (int p = 0; p < ACH; ++p) {
      const int c = p * 256 + tid;
      const int m = min(m0 + c / CPR, mlast), k = min(k0 + (c % CPR) * 8, klast);
      pa[p] = ld16(A + (long)m * lda + k);
    }
#pragma unroll
    for (int p = 0; p < BCH; ++p) {
      const int c = p * 256 + tid;
      const int n = min(n0 + c / CPR, nlast), k = min(k0 + (c % CPR) * 8, klast);
      pb[p] = ld16(Wb + (long)n * K + k);
    }
  };
  auto store2 = [&](int stg, int buf, const u32x4* pa, const u32x4* pb) {
    const int k0 = stg * KS;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int p = 0; p < ACH; ++p) {
      const int c = p * 256 + tid;
      st16(&Sm[buf][c / CPR][(c % CPR) * 8], k0 + (c % CPR) * 8 < K ? pa[p] : z);
    }
#pragma unroll
    for (int p = 0; p < BCH; ++p) {
      const int c = p * 256 + tid;
      st16(&Sm[buf][MT + c / CPR][(c % CPR) * 8], k0 + (c % CPR) * 8 < K ? pb[p] : z);
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < KS; kk += 32) {
      half8 af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const half8*>(&Sm[buf][wm0 + 16 * i + fr][kk + fk]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[j] = *reinterpret_cast<const half8*>(&Sm[buf][MT + wn0 + 16 * j + fr][kk + fk]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };
  // ring: at stage r, qa/qb[r & 1] hold stage r (already in LDS buffer
  // r & 1) and qa/qb[(r + 1) & 1] hold stage r + 1 (in flight)
  const int nrel = st1 - st0;
  if (nrel > 0) {
    load2(st0, qa[0], qb[0]);
    if (nrel > 1) load2(st0 + 1, qa[1], qb[1]);
    store2(st0, 0, qa[0], qb[0]);
    __syncthreads();
  }
  int r0 = 0;
  for (; r0 + 4 <= nrel; r0 += 2) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int r = r0 + d;
      load2(st0 + r + 2, qa[d], qb[d]);
      __builtin_amdgcn_sched_barrier(0);
      compute(d);
      __builtin_amdgcn_sched_barrier(0);
      store2(st0 + r + 1, d ^ 1, qa[d ^ 1], qb[d ^ 1]);
      __syncthreads();
    }
  }
  for (; r0 < nrel; r0 += 2) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int r = r0 + d;
      if (r < nrel) {
        if (r + 2 < nrel) load2(st0 + r + 2, qa[d], qb[d]);
        compute(d);
        if (r + 1 < nrel) store2(st0 + r + 1, d ^ 1, qa[d ^ 1], qb[d ^ 1]);
        __syncthreads();
      }
    }
  }
  } else if constexpr (!PIPE) {
  if (st0 < st1) {
    load(st0);
    store(0);
    __syncthreads();
  }
  int buf = 0;
  for (int stg = st0; stg < st1; ++stg) {
    const bool more = stg + 1 < st1;
    if (more) load(stg + 1);
#pragma unroll
    for (int kk = 0; kk < KS; kk += 32) {
      half8 af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const half8*>(&Sm[buf][wm0 + 16 * i + fr][kk + fk]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[j] = *reinterpret_cast<const half8*>(&Sm[buf][MT + wn0 + 16 * j + fr][kk + fk]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  } else {
  // Software pipeline: the fragments of stage s + 1 are read from LDS while
  // the MFMAs of stage s run, stage s + 2 waits in registers and is written
  // to LDS after them, and stage s + 3 is in flight from global memory.
  constexpr int KH = KS / 32;
  half8 fa[2][KH][TM], fb[2][KH][TN];
  auto read_frags = [&](int buf, half8 (*pa)[TM], half8 (*pb)[TN]) {
#pragma unroll
    for (int h = 0; h < KH; ++h) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        pa[h][i] = *reinterpret_cast<const half8*>(&Sm[buf][wm0 + 16 * i + fr][32 * h + fk]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        pb[h][j] = *reinterpret_cast<const half8*>(&Sm[buf][MT + wn0 + 16 * j + fr][32 * h + fk]);
    }
  };
  auto mfmas = [&](half8 (*pa)[TM], half8 (*pb)[TN]) {
#pragma unroll
    for (int h = 0; h < KH; ++h)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[h][i], pb[h][j], acc[i][j], 0, 0, 0);
  };
  const int nrel = st1 - st0;
  if (nrel > 0) {
    load(st0);
    store(0);
    if (nrel > 1) load(st0 + 1);
    __syncthreads();
    if (nrel > 1) store(1);
    read_frags(0, fa[0], fb[0]);
    if (nrel > 2) load(st0 + 2);
    __syncthreads();
  }
  for (int r0 = 0; r0 < nrel; r0 += 2) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = r0 + p;
      if (r < nrel) {
        if (r + 1 < nrel) read_frags((r + 1) & 1, fa[p ^ 1], fb[p ^ 1]);
        mfmas(fa[p], fb[p]);
        if (r + 2 < nrel) store(r & 1);
        if (r + 3 < nrel) load(st0 + r + 3);
        __syncthreads();
      }
    }
  }
  }

  if constexpr (sizeof(Sm) >= MT * (NT + 4) * 4)
    mm_epilogue_lds<TM, TN, MT, NT>(a, sg, acc, ks_id, n0, m0, wm0, wn0, lane, reinterpret_cast<float*>(&Sm[0][0][0]));
  else
    mm_epilogue<TM, TN>(a, sg, acc, ks_id, n0, m0, wm0, wn0, lane);
}

// ------------------------------------------------------- LDS-DMA variant
// The same tile and epilogue, with each stage going from global memory
// straight into LDS (global_load_lds_dwordx4 writes each lane's 16 bytes at
// M0 + 16 * lane): no staging registers and no LDS write instructions, three
// stages in an LDS ring, one of them in flight while another is multiplied.
// The loads are issued from inline assembly and their waits placed by hand:
// for the compiler's own form of the load, the waitcnt pass drains every
// pending LDS DMA before any LDS read, which would leave nothing in flight.
// The main loop issues no other vector-memory instruction, so the counts
// below are exact.  Requires K to be a multiple of KS.
//
// LDS layout per stage: the A rows, then the W rows, KS halves each with no
// padding (a DMA instruction fills 1 KB contiguously).  Fragment reads take
// 16 rows at one k chunk; rows 16 apart would share banks, so chunk c of
// row r is stored at position c ^ swz(r), which spreads those 16 reads over
// all 64 banks.
__device__ inline void dma16(const half_t* g, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory");
}
template <int N>
__device__ inline void wait_vm() {   // vmcnt <= N; lgkmcnt and expcnt unconstrained
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
template <int CPR>
__device__ inline int swz(int r) {
  return CPR == 4 ? ((r >> 2) & 3) : CPR == 8 ? ((r >> 1) & 7) : (r & 15);
}
// NW = 4: waves as 2 x 2, each (16 TM) x (16 TN); NW = 8 (K loop 4): waves
// as 2 x 4, each (16 TM) x (8 TN): two waves per SIMD on the same tile.
template <int TM, int TN, int KS, int NW>
__global__ __launch_bounds__(64 * NW) void k_mm_dma(ProjArgs a) {
  constexpr int MT = 32 * TM, NT = 32 * TN, CPR = KS / 8, KH = KS / 32;
  constexpr int WC = NW / 2;               // wave columns
  constexpr int BN = 2 * TN / WC;          // 16 x 16 blocks per wave along N
  constexpr int SLOTS = (MT + NT) * CPR;   // 16-byte slots per stage
  // every wave issues the same whole number of DMA instructions per stage (so
  // the wait counts are exact); lanes past the stage's slots fill padding
  constexpr int NIW = (SLOTS + 64 * NW - 1) / (64 * NW);   // DMA instructions per wave and stage
  constexpr int SLOTS_PAD = NIW * 64 * NW;
  constexpr int ASL = MT * CPR;            // slots of the A rows
  static_assert((2 * TN) % WC == 0, "whole blocks per wave");
  __shared__ __attribute__((aligned(1024))) half_t L[3][SLOTS_PAD * 8];

  const int n_tiles = a.tile0[a.nseg];
  const int total = n_tiles * a.m_tiles * a.split;
  const int per_xcd = (total + 7) / 8;
  const int lin = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (lin >= total) return;
  const int ks_id = lin % a.split;
  const int m_tile = (lin / a.split) % a.m_tiles;
  const int n_tile = lin / (a.split * a.m_tiles);
  Seg sg = a.seg[0];
  int t0 = 0;
#pragma unroll
  for (int i = 1; i < MAX_SEGS; ++i)
    if (i < a.nseg && n_tile >= a.tile0[i]) {
      sg = a.seg[i];
      t0 = a.tile0[i];
    }
  const int n0 = sg.row0 + (n_tile - t0) * NT;
  const int m0 = m_tile * MT;
  const bool own = sg.W != nullptr;
  const int K = own ? sg.K : a.K;
  const half_t* Wb = own ? sg.W - (long)sg.row0 * K : a.W;
  const half_t* A = reinterpret_cast<const half_t*>(sg.act) + sg.act_off;
  const int lda = sg.ld_act;
  const int nst = K / KS;
  const int st0 = (int)((long)nst * ks_id / a.split);
  const int st1 = (int)((long)nst * (ks_id + 1) / a.split);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / WC) * 16 * TM, wn0 = (wave % WC) * 16 * BN;

  // source of each lane in this wave's DMA instructions, at stage 0; rows
  // past the end read the last row (their outputs are not stored)
  const half_t* src[NIW];
#pragma unroll
  for (int q = 0; q < NIW; ++q) {
    const int S = (q * NW + wave) * 64 + lane;
    if (S < ASL) {
      const int r = S / CPR, c = (S % CPR) ^ swz<CPR>(r);
      src[q] = A + (long)min(m0 + r, a.M - 1) * lda + c * 8;
    } else if (S < SLOTS) {
      const int r = (S - ASL) / CPR, c = ((S - ASL) % CPR) ^ swz<CPR>(r);
      src[q] = Wb + (long)min(n0 + r, sg.row1 - 1) * K + c * 8;
    } else {   // padding slot: any valid row chunk of A
      src[q] = A + (long)min(m0, a.M - 1) * lda;
    }
  }
  const unsigned lds0 = (unsigned)(uintptr_t)&L[0][0];
  auto issue = [&](int stg, int slot) {
#pragma unroll
    for (int q = 0; q < NIW; ++q)
      dma16(src[q] + (long)stg * KS,
            __builtin_amdgcn_readfirstlane(lds0 + slot * SLOTS_PAD * 16 + (q * NW + wave) * 1024));
  };
  int aoff[KH][TM], boff[KH][BN];   // byte offsets of this lane's fragments in a stage
#pragma unroll
  for (int h = 0; h < KH; ++h) {
    const int c = 4 * h + (lane >> 4);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm0 + 16 * i + (lane & 15);
      aoff[h][i] = (r * CPR + (c ^ swz<CPR>(r))) * 16;
    }
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      const int r = wn0 + 16 * j + (lane & 15);
      boff[h][j] = (ASL + r * CPR + (c ^ swz<CPR>(r))) * 16;
    }
  }
  floatx4 acc[TM][BN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < BN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int slot) {
    const char* Lb = reinterpret_cast<const char*>(&L[slot][0]);
#pragma unroll
    for (int h = 0; h < KH; ++h) {
      half8 af[TM], bf[BN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const half8*>(Lb + aoff[h][i]);
#pragma unroll
      for (int j = 0; j < BN; ++j) bf[j] = *reinterpret_cast<const half8*>(Lb + boff[h][j]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < BN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };
  // stage r lives in slot r % 3; at the top of stage r, stages r and r + 1
  // are in flight (NIW instructions each per wave)
  const int nrel = st1 - st0;
  if (nrel > 0) issue(st0, 0);
  if (nrel > 1) issue(st0 + 1, 1);
  int r0 = 0;
  for (; r0 + 5 <= nrel; r0 += 3) {
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      wait_vm<NIW>();     // this wave's part of stage r0 + d has landed
      __syncthreads();    // ... every wave's; and every wave is done with slot (d + 2) % 3
      issue(st0 + r0 + d + 2, (d + 2) % 3);
      compute(d);
    }
  }
  for (; r0 < nrel; r0 += 3) {
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      const int r = r0 + d;
      if (r < nrel) {
        if (r + 1 < nrel) wait_vm<NIW>();
        else wait_vm<0>();
        __syncthreads();
        if (r + 2 < nrel) issue(st0 + r + 2, (d + 2) % 3);
        compute(d);
      }
    }
  }
  wait_vm<0>();
  if constexpr (sizeof(L) >= MT * (NT + 4) * 4)
    mm_epilogue_lds<TM, BN, MT, NT>(a, sg, acc, ks_id, n0, m0, wm0, wn0, lane, reinterpret_cast<float*>(&L[0][0]));
  else if constexpr (sizeof(L) >= 64 * (NT + 4) * 4 && MT % 64 == 0)
    mm_epilogue_lds<TM, BN, MT, NT, (sizeof(L) >= 128 * (NT + 4) * 4 && MT % 128 == 0) ? 128 : 64>(
        a, sg, acc, ks_id, n0, m0, wm0, wn0, lane, reinterpret_cast<float*>(&L[0][0]));
  else
    mm_epilogue<TM, BN>(a, sg, acc, ks_id, n0, m0, wm0, wn0, lane);
}

// ------------------------------------------------------- LDS-DMA ring
// k_mm_dma with a deeper ring: `nslot` stages (a launch argument; dynamic
// LDS of nslot * (MT + NT) * KS * 2 bytes), nslot - 1 of them in flight
// while one is multiplied.  A decode projection (M <= 256) streams each
// weight once; what bounds it is how many bytes each CU keeps in flight
// against the memory latency, not the MFMA rate, and a three-slot ring
// keeps too few (about 20 GB/s per CU at M = 64).  At the top of stage r
// the stages r .. r + nslot - 2 are in flight; once the last stage has been
// issued, one full wait covers the rest, which are then multiplied out with
// no further barrier.
// vmcnt <= stages * NIW for a runtime stage count (the count is an
// instruction immediate; the branch is on a workgroup-uniform value)
template <int NIW, int K>
__device__ inline void wait_k() {   // vmcnt <= K * NIW, or less where that exceeds the field
  constexpr int k = K * NIW <= 63 ? K : 63 / NIW;
  wait_vm<k * NIW>();
}
template <int NIW>
__device__ inline void wait_stages(int stages) {
  switch (stages) {
    case 0: wait_vm<0>(); break;
    case 1: wait_k<NIW, 1>(); break;
    case 2: wait_k<NIW, 2>(); break;
    case 3: wait_k<NIW, 3>(); break;
    case 4: wait_k<NIW, 4>(); break;
    case 5: wait_k<NIW, 5>(); break;
    case 6: wait_k<NIW, 6>(); break;
    default: wait_k<NIW, 7>(); break;
  }
}
constexpr int RING_MAX_SLOTS = 9;   // stages - 2 <= 7 in flight behind the one waited for

template <int TM, int TN, int KS>
__global__ __launch_bounds__(256) void k_mm_ring(ProjArgs a, int nslot) {
  constexpr int NW = 4;
  constexpr int MT = 32 * TM, NT = 32 * TN, CPR = KS / 8, KH = KS / 32;
  constexpr int SLOTS = (MT + NT) * CPR;
  constexpr int NIW = SLOTS / (64 * NW);
  constexpr int ASL = MT * CPR;
  static_assert(SLOTS % (64 * NW) == 0, "whole DMA instructions per wave");
  extern __shared__ __attribute__((aligned(1024))) half_t Ld[];

  const int n_tiles = a.tile0[a.nseg];
  const int total = n_tiles * a.m_tiles * a.split;
  const int per_xcd = (total + 7) / 8;
  const int lin = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (lin >= total) return;
  const int ks_id = lin % a.split;
  const int m_tile = (lin / a.split) % a.m_tiles;
  const int n_tile = lin / (a.split * a.m_tiles);
  Seg sg = a.seg[0];
  int t0 = 0;
#pragma unroll
  for (int i = 1; i < MAX_SEGS; ++i)
    if (i < a.nseg && n_tile >= a.tile0[i]) {
      sg = a.seg[i];
      t0 = a.tile0[i];
    }
  const int n0 = sg.row0 + (n_tile - t0) * NT;
  const int m0 = m_tile * MT;
  const bool own = sg.W != nullptr;
  const int K = own ? sg.K : a.K;
  const half_t* Wb = own ? sg.W - (long)sg.row0 * K : a.W;
  const half_t* A = reinterpret_cast<const half_t*>(sg.act) + sg.act_off;
  const int lda = sg.ld_act;
  const int nst = K / KS;
  const int st0 = (int)((long)nst * ks_id / a.split);
  const int st1 = (int)((long)nst * (ks_id + 1) / a.split);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave >> 1) * 16 * TM, wn0 = (wave & 1) * 16 * TN;

  const half_t* src[NIW];
#pragma unroll
  for (int q = 0; q < NIW; ++q) {
    const int S = (q * NW + wave) * 64 + lane;
    if (S < ASL) {
      const int r = S / CPR, c = (S % CPR) ^ swz<CPR>(r);
      src[q] = A + (long)min(m0 + r, a.M - 1) * lda + c * 8;
    } else {
      const int r = (S - ASL) / CPR, c = ((S - ASL) % CPR) ^ swz<CPR>(r);
      src[q] = Wb + (long)min(n0 + r, sg.row1 - 1) * K + c * 8;
    }
  }
  const unsigned lds0 = (unsigned)(uintptr_t)&Ld[0];
  auto issue = [&](int stg, int slot) {
#pragma unroll
    for (int q = 0; q < NIW; ++q)
      dma16(src[q] + (long)stg * KS,
            __builtin_amdgcn_readfirstlane(lds0 + slot * SLOTS * 16 + (q * NW + wave) * 1024));
  };
  int aoff[KH][TM], boff[KH][TN];
#pragma unroll
  for (int h = 0; h < KH; ++h) {
    const int c = 4 * h + (lane >> 4);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm0 + 16 * i + (lane & 15);
      aoff[h][i] = (r * CPR + (c ^ swz<CPR>(r))) * 16;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn0 + 16 * j + (lane & 15);
      boff[h][j] = (ASL + r * CPR + (c ^ swz<CPR>(r))) * 16;
    }
  }
  floatx4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int slot) {
    const char* Lb = reinterpret_cast<const char*>(Ld) + slot * SLOTS * 16;
#pragma unroll
    for (int h = 0; h < KH; ++h) {
      half8 af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const half8*>(Lb + aoff[h][i]);
#pragma unroll
      for (int j = 0; j < TN; ++j) bf[j] = *reinterpret_cast<const half8*>(Lb + boff[h][j]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };
  const int nrel = st1 - st0;
  const int pre = min(nrel, nslot - 1);
  for (int r = 0; r < pre; ++r) issue(st0 + r, r);
  // steady state: stage r + nslot - 1 is issued into the slot stage r - 1 used
  int r = 0, slot = 0, fill = nslot - 1;
  for (; r + nslot - 1 < nrel; ++r) {
    wait_stages<NIW>(nslot - 2);   // stage r has landed (this wave's part)
    __syncthreads();               // every wave's; every wave is done with stage r - 1's slot
    issue(st0 + r + nslot - 1, fill);
    compute(slot);
    slot = slot + 1 == nslot ? 0 : slot + 1;
    fill = fill + 1 == nslot ? 0 : fill + 1;
  }
  // tail: nothing more to issue
  wait_vm<0>();
  __syncthreads();
  for (; r < nrel; ++r) {
    compute(slot);
    slot = slot + 1 == nslot ? 0 : slot + 1;
  }
  const bool lds_epi = (int)(nslot * SLOTS * 16) >= MT * (NT + 4) * 4;
  if (lds_epi)
    mm_epilogue_lds<TM, TN, MT, NT>(a, sg, acc, ks_id, n0, m0, wm0, wn0, lane, reinterpret_cast<float*>(Ld));
  else
    mm_epilogue<TM, TN>(a, sg, acc, ks_id, n0, m0, wm0, wn0, lane);
}

// Fixed-order sum of the split-K partials, then the segment's epilogue.
__global__ __launch_bounds__(256) void k_mm_reduce(ProjArgs a) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const long total = (long)a.M * a.total_rows;
  if (idx >= total) return;
  const int m = (int)(idx / a.total_rows);
  const int n = (int)(idx % a.total_rows);
  float v = 0.f;
  for (int s = 0; s < a.split; ++s) v += a.part[(long)s * total + idx];
  const Seg sg = pick_seg(a, n);
  if (n < sg.row1) epi_store(sg, n - sg.row0, m, v);
}

// Union mask of the sparse path when the key projection runs on MFMA:
// computed afterwards from the stored pre-activations.
__global__ void k_pre_mask(const float* pre, int ld, int M, int F, unsigned char* mask) {
  const int f = blockIdx.x * blockDim.x + threadIdx.x;
  if (f >= F) return;
  bool any = false;
  for (int m = 0; m < M; ++m) any |= pre[(long)m * ld + f] > 0.0f;
  mask[f] = any ? 1 : 0;
}

// Tile plan of a launch with TM x TN blocks of 16 x 16 per wave (tile
// 32 TM x 32 TN) and KS-deep stages: column tiles per segment, M tiles, and
// the K split (split_req 0: about 1.5 workgroups per CU when the tiles are
// fewer than the CUs, at least 4 stages per range, within the partial-sum
// buffer).
int mm_plan(ProjArgs& a, int total_rows, int tm, int tn, int ks, int split_req, int64_t part_floats) {
  const int NT = 32 * tn;
  const int MT = 32 * tm;
  a.tile0[0] = 0;
  int max_nst = 1;
  for (int i = 0; i < a.nseg; ++i) {
    const Seg& s = a.seg[i];
    const int K = s.W ? s.K : a.K;
    if (K % 32 != 0 || K <= 0) return -1;
    if (s.row1 <= s.row0) return -1;
    a.tile0[i + 1] = a.tile0[i] + (s.row1 - s.row0 + NT - 1) / NT;
    const int nst = (K + ks - 1) / ks;
    max_nst = max_nst > nst ? max_nst : nst;
  }
  for (int i = a.nseg + 1; i <= MAX_SEGS; ++i) a.tile0[i] = a.tile0[a.nseg];
  a.m_tiles = (a.M + MT - 1) / MT;
  a.total_rows = total_rows;
  const int tiles = a.tile0[a.nseg] * a.m_tiles;
  int split = 1;
  if (a.part) {
    if (split_req > 0) {
      split = split_req;
    } else if (tiles < 256) {
      split = (384 + tiles - 1) / tiles;
      if (split > max_nst / 4) split = max_nst / 4;
    }
    if (split > max_nst) split = max_nst;
    while (split > 1 && (int64_t)split * a.M * total_rows > part_floats) --split;
    if (split < 1) split = 1;
  }
  a.split = split;
  return tiles * split;
}

// LDS bytes of a k_mm instantiation (two stage buffers of A and W rows)
static constexpr int mm_lds_bytes(int tm, int tn, int ks) { return 2 * 32 * (tm + tn) * (ks + MM_PAD) * 2; }

template <int TM, int TN, int PIPE>
static void mm_launch_p(int ks, dim3 grid, hipStream_t st, const ProjArgs& a) {
  if constexpr (TM >= 2) {
    if (ks == 32) {
      hipLaunchKernelGGL((k_mm<TM, TN, 32, PIPE>), grid, dim3(256), 0, st, a);
      return;
    }
  }
  if constexpr (mm_lds_bytes(TM, TN, 128) <= 81920 && !(PIPE && TM + TN > 4)) {
    if (ks == 128) {
      hipLaunchKernelGGL((k_mm<TM, TN, 128, PIPE>), grid, dim3(256), 0, st, a);
      return;
    }
  }
  hipLaunchKernelGGL((k_mm<TM, TN, 64, PIPE>), grid, dim3(256), 0, st, a);
}

// LDS bytes of a k_mm_dma instantiation (three unpadded stages)
static constexpr int mm_dma_lds_bytes(int tm, int tn, int ks) { return 3 * 32 * (tm + tn) * ks * 2; }

template <int TM, int TN, int NW>
static void mm_launch_dma(int ks, dim3 grid, hipStream_t st, const ProjArgs& a) {
  if constexpr (TM >= 2 && (TM + TN) % (NW / 2) == 0) {
    if (ks == 32) {
      hipLaunchKernelGGL((k_mm_dma<TM, TN, 32, NW>), grid, dim3(64 * NW), 0, st, a);
      return;
    }
  }
  if constexpr (mm_dma_lds_bytes(TM, TN, 128) <= 98304) {
    if (ks == 128) {
      hipLaunchKernelGGL((k_mm_dma<TM, TN, 128, NW>), grid, dim3(64 * NW), 0, st, a);
      return;
    }
  }
  hipLaunchKernelGGL((k_mm_dma<TM, TN, 64, NW>), grid, dim3(64 * NW), 0, st, a);
}

// Ring depth of K loops 5 (about 144 KB of LDS: one workgroup per CU) and
// 6 (about 72 KB: two per CU); 0 when fewer than three stages fit.
static constexpr int ring_stage_bytes(int tm, int tn, int ks) { return 32 * (tm + tn) * ks * 2; }
static int ring_slots(int tm, int tn, int ks, int pipe) {
  const int budget = pipe == 5 ? 147456 : 73728;
  int n = budget / ring_stage_bytes(tm, tn, ks);
  if (n > RING_MAX_SLOTS) n = RING_MAX_SLOTS;
  return n >= 3 ? n : 0;
}

template <int TM, int TN>
static void mm_launch_ring(int ks, int pipe, dim3 grid, hipStream_t st, const ProjArgs& a) {
  const int n = ring_slots(TM, TN, ks, pipe);
  const size_t lds = (size_t)n * ring_stage_bytes(TM, TN, ks);
  if (ks == 128)
    hipLaunchKernelGGL((k_mm_ring<TM, TN, 128>), grid, dim3(256), lds, st, a, n);
  else
    hipLaunchKernelGGL((k_mm_ring<TM, TN, 64>), grid, dim3(256), lds, st, a, n);
}

template <int TM, int TN>
static void mm_launch(int ks, int pipe, dim3 grid, hipStream_t st, const ProjArgs& a) {
  if (pipe == 5 || pipe == 6) {
    mm_launch_ring<TM, TN>(ks, pipe, grid, st, a);
    return;
  }
  if (pipe == 3) {
    mm_launch_dma<TM, TN, 4>(ks, grid, st, a);
    return;
  }
  if constexpr (TN % 2 == 0 && (TM + TN) % 2 == 0) {
    if (pipe == 4) {
      mm_launch_dma<TM, TN, 8>(ks, grid, st, a);
      return;
    }
  }
  if constexpr (TM + TN <= 6) {
    if (pipe == 1) {
      mm_launch_p<TM, TN, 1>(ks, grid, st, a);
      return;
    }
    if (pipe == 2) {
      mm_launch_p<TM, TN, 2>(ks, grid, st, a);
      return;
    }
  }
  mm_launch_p<TM, TN, 0>(ks, grid, st, a);
}

static bool mm_cfg_ok(int tm, int tn, int ks, int pipe) {
  if (pipe < 0 || pipe > 6) return false;
  if (pipe == 5 || pipe == 6) {   // LDS-DMA ring
    if (!((tm == 1 || tm == 2 || tm == 4) && (tn == 2 || tn == 4))) return false;
    return (ks == 64 || ks == 128) && ring_slots(tm, tn, ks, pipe) >= 3;
  }
  if (pipe == 4) {   // eight waves: N blocks split over four wave columns
    if (tn == 8 && tm == 8) return ks == 32;   // 256 x 256 tiles: eight waves of 128 x 64, 96 KB of LDS
    if (tn == 10) return tm == 8 && ks == 32;   // 256 x 320 tiles: eight waves of 128 x 80, 120 KB of LDS
    if (tn == 8)      // 256-wide tiles, 64-deep stages (three of them fill up to 144 KB of LDS)
      return (tm == 2 || tm == 4) && ks == 64;
    if (!((tm == 2 || tm == 4) && (tn == 2 || tn == 4))) return false;
    if (ks == 32) return (tm + tn) % 4 == 0;
    return (ks == 64 || ks == 128) && mm_dma_lds_bytes(tm, tn, ks) <= 98304;
  }
  if (pipe == 3) {
    if (tm == 2 && tn == 5) return ks == 64;   // 64 x 160 tiles (see mm_choose)
    if (tm == 4 && tn == 1) return ks == 64 || ks == 128;   // 128 x 32 tiles (see mm_choose)
    if (tm == 4 && tn == 5) return ks == 64;   // 128 x 160 tiles, 108 KB of LDS (see mm_choose)
    if (!((tm == 1 || tm == 2 || tm == 4) && (tn == 2 || tn == 4))) return false;
    if (ks == 32) return tm >= 2;
    return (ks == 64 || ks == 128) && mm_dma_lds_bytes(tm, tn, ks) <= 98304;
  }
  if (pipe && (tm + tn > 6 || (ks == 128 && tm + tn > 4))) return false;
  if (!((tm == 1 || tm == 2 || tm == 4) && (tn == 2 || tn == 4))) return false;
  if (ks == 32) return tm >= 2;
  if (ks == 128) return mm_lds_bytes(tm, tn, 128) <= 81920;
  return ks == 64;
}

// Default plan by problem shape, from sweeps of (tm, tn, ks, pipe, split) on
// MI355X: the 2.9B and 7.2B projections at M = 64, 256 and 512 with the
// weights streamed from HBM (rotated over six copies), then the 2.9B model's
// own projections chosen one at a time on whole graph-replayed decode steps
// (B = 64, 256; the 7.2B model at B = 256) and 512- and 2048-token prefill
// chunks.  At M <= 64: 64 x 64 tiles with 128-deep stages on the DMA loop,
// split 6 for the narrow outputs (W_o, value; their partials go to the next
// LayerNorm) and no split for the key (3.63 -> 3.50 ms per 2.9B B = 64 step).  A kernel timed alone can
// rank plans differently from the step it runs in (the 64 x 160 key tiles
// are 12 % faster alone and only even in the step), so the step decides.  "Narrow" outputs are one model width (value,
// output projection), "head" the vocabulary, "wide" the rest (key, input
// projection, adapters' second stage, whose K is an adapter rank).
// split 0 = automatic.
struct MmPlan {
  int tm, tn, ks, pipe, split;
};
static MmPlan mm_choose(const ProjArgs& a, int total_rows) {
  const int M = a.M, N = total_rows;
  int K = a.K;
  for (int i = 0; i < a.nseg; ++i)
    if (a.seg[i].W && a.seg[i].K > K) K = a.seg[i].K;
  if (M <= 32) {
    // 32 x 64 tiles on the DMA loop, W_o and the value split 6 (their
    // partials go to the next LayerNorm), the input projection split 4; the
    // adapters' second stage stays on the register-staged loop (whole 2.9B
    // decode steps at B = 8 / 16 / 32: 7.2 / 7.5 / 6.6 % faster)
    if (N >= 32768) return {1, 4, 64, 3, 0};
    if (N <= 4096) return {1, 2, 128, 3, 6};
    if (K < 1024) return {1, 2, 128, 0, 0};
    return a.nseg == 1 ? MmPlan{1, 2, 64, 3, 0} : MmPlan{1, 2, 128, 3, 4};
  }
  if (N <= 4096) {                                   // narrow
    if (K >= 8192) {                                 // channel-mix value
      if (K >= 16384) return M > 64 && M <= 256 ? MmPlan{4, 4, 64, 4, 3} : MmPlan{4, 4, 64, 0, 6};
      if (M <= 64) return {2, 2, 128, 3, 6};
      // 65 - 128 rows: 128 x 32 tiles in three K ranges, 240 workgroups each
      // reading its weight columns once (2.9B: 128-token prefill 4.50 -> 4.40
      // ms, B = 128 steps 4.80 -> 4.74 ms; slower at 256 rows)
      if (M <= 128) return {4, 1, 128, 3, 3};
      if (M <= 256) return {4, 4, 64, 4, 6};
      // above 1024 rows: 256 x 256 tiles, three K ranges (2048-token prefill 0.5 % faster)
      // 257 - 1024 rows: 128 x 160 tiles in four K ranges (one round of 256
      // workgroups at 512 rows; 512-token prefill 8.14 -> 7.84 ms)
      return M <= 1024 ? MmPlan{4, 5, 64, 3, 4} : MmPlan{8, 8, 32, 4, 3};
    }
    if (M <= 64) return {2, 2, 128, 3, 6};
    // 129 - 256 rows: 64 x 128 tiles in two K ranges where they make one round
    // of 192 - 256 workgroups (7.2B W_o at B = 256: 256; steps 10.83 -> 10.67 ms)
    if (M > 128 && M <= 256) {
      const long t = (long)(M + 63) / 64 * ((N + 127) / 128) * 2;
      if (t >= 192 && t <= 256) return {2, 4, 64, 4, 2};
    }
    // 513 - 1024 rows: 128 x 160 tiles in two K ranges, one round at 1024 rows
    // (1024-token prefill 14.44 -> 14.05 ms; no gain at 512 or 2048 rows)
    if (M > 512 && M <= 1024) return {4, 5, 64, 3, 2};
    return M <= 256 ? MmPlan{2, 2, 64, 4, 0} : MmPlan{2, 4, 64, 4, 0};
  }
  if (N >= 32768)   // head (193 - 256 rows: 256 x 256 tiles, one per CU for a 65536-token vocabulary)
    return M <= 64 ? MmPlan{2, 4, 64, 3, 0} : M <= 192 ? MmPlan{4, 8, 64, 4, 0} : M <= 256 ? MmPlan{8, 8, 32, 4, 0}
                                                                                 : MmPlan{4, 4, 64, 0, 0};
  const bool rank_k = K < 1024;                      // adapters' second stage
  if (M <= 64) {
    if (rank_k) return {1, 2, 128, 0, 0};
    // the key: one K range (no split, so no reduction launch before its ReLU^2)
    return N <= 8192 ? MmPlan{1, 2, 128, 3, 0} : MmPlan{2, 2, 128, 3, 1};
  }
  if (M <= 256) {
    if (rank_k) return {2, 2, 64, 2, 0};
    if (K >= 4096) return N >= 16384 ? MmPlan{4, 4, 64, 4, 0} : MmPlan{4, 2, 64, 4, 0};
    // the key on 64 x 128 tiles with one K range while they fit one round of
    // 256 CUs (2.9B: up to 192 rows; 38 -> 29 us at 128 and 192 rows), and
    // up to 128 rows the input projection on 64 x 64 tiles with 128-deep
    // stages (40 -> 32 us): whole 128-token prefill 4.93 -> 4.37 ms, B = 128
    // decode steps 5.40 -> 4.93 ms
    // 65 - 128 rows: the key on 128 x 128 tiles in three K ranges (240
    // workgroups, each operand read once per tile pair) plus the reduction
    // launch beats one K range (2.9B: 128-token prefill 4.41 -> 4.31 ms, B = 128
    // steps 4.73 -> 4.66 ms)
    if (a.nseg == 1 && M > 64 && M <= 128 && N >= 8192) return {4, 4, 64, 4, 3};
    if (a.nseg == 1 && (long)(M + 63) / 64 * ((N + 127) / 128) <= 256) return {2, 4, 64, 3, 1};
    if (M <= 128 && a.nseg > 1) return {2, 2, 128, 3, 0};
    // one segment: 64 x 160 tiles when they fill the CUs in fewer column-widths
    // of rounds than 64 x 64 tiles (2.9B key at M = 256: 256 tiles, one per CU,
    // instead of 640, which leave half the CUs a third round)
    if (a.nseg == 1 && K % 64 == 0) {
      const long mt = (M + 63) / 64;
      const long r2 = ((N + 63) / 64 * mt + 255) / 256, r5 = ((N + 159) / 160 * mt + 255) / 256;
      if (r5 * 160 < r2 * 64) return {2, 5, 64, 3, 0};
    }
    return N <= 8192 ? MmPlan{4, 2, 64, 4, 0} : MmPlan{2, 2, 64, 1, 0};
  }
  if (rank_k) return {2, 2, 32, 2, 0};
  // above 1024 rows: 256 x 320 tiles where they make one round of 192 - 256
  // workgroups (2.9B at 2048 rows: the key 256 tiles, the input projection
  // 224; whole 2048-token prefills 24.09 -> 21.95 ms; at 1024 rows half the
  // CUs would idle)
  if (M > 1024 && K % 32 == 0) {
    long t = 0;
    for (int i = 0; i < a.nseg; ++i) t += (a.seg[i].row1 - a.seg[i].row0 + 319) / 320;
    t *= (M + 255) / 256;
    if (t >= 192 && t <= 256) return {8, 10, 32, 4, 1};
  }
  if (K >= 4096) return N >= 10240 ? MmPlan{2, 4, 32, 1, 1} : MmPlan{4, 2, 64, 2, 0};
  // the key (one segment), one K range: up to 1024 rows 128 x 160 tiles (2.9B at
  // 512 rows: 256 of them; 512- and 1024-token prefills 2.2 and 1.7 % faster
  // than 128 x 256 tiles), above that 128 x 256 tiles where 256 x 320 ones do
  // not make one round
  if (N >= 10240 && a.nseg == 1 && K % 64 == 0) return M <= 1024 ? MmPlan{4, 5, 64, 3, 1} : MmPlan{4, 8, 64, 4, 1};
  if (N >= 10240) return M <= 1024 ? MmPlan{2, 2, 64, 4, 0} : MmPlan{4, 4, 64, 4, 0};
  return {4, 2, 64, 4, 0};
}

hipError_t launch_gemm_cfg(ProjArgs a, int total_rows, int64_t part_floats, int tm, int tn, int ks,
                           int split, hipStream_t st, int* deferred) {
  if (deferred) *deferred = 0;
  // ks >= 1000: pipelined loop number ks / 1000 with stage depth ks % 1000
  int pipe = 0;
  if (ks >= 1000) {
    pipe = ks / 1000;
    ks %= 1000;
  }
  if (tm <= 0 || tn <= 0 || ks <= 0) {
    const MmPlan p = mm_choose(a, total_rows);
    tm = p.tm; tn = p.tn; ks = p.ks; pipe = p.pipe;
    if (split <= 0) split = p.split;
  }
  if (!mm_cfg_ok(tm, tn, ks, pipe)) return hipErrorInvalidValue;
  if (pipe >= 3)   // the DMA loops need whole stages: otherwise a register-staged loop
    for (int i = 0; i < a.nseg; ++i)
      if ((a.seg[i].W ? a.seg[i].K : a.K) % ks != 0) {
        if (tn == 1 || tn == 5 || tn == 8 || tn == 10) tn = tn == 1 ? 2 : 4;   // 32-, 160-, 256-, 320-wide: DMA only
        if (tm == 8) tm = 4;
        if (!mm_cfg_ok(tm, tn, ks, 2) && !mm_cfg_ok(tm, tn, ks, 0)) ks = 64;   // register loops' LDS limits
        pipe = mm_cfg_ok(tm, tn, ks, 2) ? 2 : 0;
      }
  if (!mm_cfg_ok(tm, tn, ks, pipe)) return hipErrorInvalidValue;
  const int items = mm_plan(a, total_rows, tm, tn, ks, split, part_floats);
  if (items < 0) return hipErrorInvalidValue;
  const dim3 grid(((items + 7) / 8) * 8);
  switch (tm * 10 + tn) {
    case 12: mm_launch<1, 2>(ks, pipe, grid, st, a); break;
    case 14: mm_launch<1, 4>(ks, pipe, grid, st, a); break;
    case 22: mm_launch<2, 2>(ks, pipe, grid, st, a); break;
    case 24: mm_launch<2, 4>(ks, pipe, grid, st, a); break;
    case 42: mm_launch<4, 2>(ks, pipe, grid, st, a); break;
    case 25: mm_launch_dma<2, 5, 4>(ks, grid, st, a); break;   // loop 3, ks 64 only
    case 45: hipLaunchKernelGGL((k_mm_dma<4, 5, 64, 4>), grid, dim3(256), 0, st, a); break;   // loop 3
    case 41:   // loop 3: 128 x 32 tiles, four waves of 64 x 16
      if (ks == 64)
        hipLaunchKernelGGL((k_mm_dma<4, 1, 64, 4>), grid, dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((k_mm_dma<4, 1, 128, 4>), grid, dim3(256), 0, st, a);
      break;
    case 28: hipLaunchKernelGGL((k_mm_dma<2, 8, 64, 8>), grid, dim3(512), 0, st, a); break;   // loop 4
    case 48: hipLaunchKernelGGL((k_mm_dma<4, 8, 64, 8>), grid, dim3(512), 0, st, a); break;   // loop 4
    case 88: hipLaunchKernelGGL((k_mm_dma<8, 8, 32, 8>), grid, dim3(512), 0, st, a); break;   // loop 4
    case 90: hipLaunchKernelGGL((k_mm_dma<8, 10, 32, 8>), grid, dim3(512), 0, st, a); break;  // 256 x 320
    default: mm_launch<4, 4>(ks, pipe, grid, st, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool can_defer = a.nseg == 1 && a.seg[0].epi == EPI_RESID && !a.seg[0].out_f16 &&
                         a.seg[0].row0 == 0 && a.seg[0].row1 == total_rows && a.seg[0].ld_out == total_rows;
  if (a.split > 1 && deferred && can_defer) {
    *deferred = a.split;
  } else if (a.split > 1) {
    const long n = (long)a.M * total_rows;
    hipLaunchKernelGGL(k_mm_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  for (int i = 0; i < a.nseg; ++i) {
    const Seg& s = a.seg[i];
    if (s.epi == EPI_PRE && s.mask) {
      const int F = s.row1 - s.row0;
      hipLaunchKernelGGL(k_pre_mask, dim3((F + 255) / 256), dim3(256), 0, st,
                         (const float*)s.out, s.ld_out, a.M, F, s.mask);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

bool gemm_cfg_ok(int tm, int tn, int ks, int pipe) { return mm_cfg_ok(tm, tn, ks, pipe); }

hipError_t launch_gemm(ProjArgs a, int total_rows, int64_t part_floats, hipStream_t st, int* deferred) {
  return launch_gemm_cfg(a, total_rows, part_floats, 0, 0, 0, 0, st, deferred);
}

// Template arguments as a trace prints them, e.g. "k_mm<4, 4, 64, 0>", for an
// M x N x K projection with the default plan.
const char* gemm_kernel_name(int M, int N, int K) {
  ProjArgs a;
  memset(&a, 0, sizeof a);
  a.M = M;
  a.K = K;
  a.nseg = 1;   // one segment of N rows
  a.seg[0].row0 = 0;
  a.seg[0].row1 = N;
  const MmPlan p = mm_choose(a, N);
  const int tm = p.tm, ks = p.ks, pipe = p.pipe;
  int tn = p.tn;
  int ep = pipe;   // as launch_gemm_cfg falls back
  if (pipe >= 3 && K % ks != 0) {
    if (tn == 5 || tn == 8) tn = 4;
    ep = mm_cfg_ok(tm, tn, ks, 2) ? 2 : 0;
  }
  static char names[4][4][3][5][32];
  char* s = names[tm == 1 ? 0 : tm == 2 ? 1 : tm == 4 ? 2 : 3][tn == 2 ? 0 : tn == 4 ? 1 : tn == 5 ? 2 : 3]
                 [ks == 32 ? 0 : ks == 64 ? 1 : 2][ep];
  if (!s[0]) {
    if (ep >= 3)
      snprintf(s, sizeof(names[0][0][0][0]), "k_mm_dma<%d, %d, %d, %d>", tm, tn, ks, ep == 4 ? 8 : 4);
    else
      snprintf(s, sizeof(names[0][0][0][0]), "k_mm<%d, %d, %d, %d>", tm, tn, ks, ep);
  }
  return s;
}
