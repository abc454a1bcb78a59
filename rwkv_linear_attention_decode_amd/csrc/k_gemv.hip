// Small-batch projections: fp16 weights [rows][K] (K contiguous) times fp32
// activations for B <= 4 rows.
//
// The RWKV-Server article (section 3) credits the decode speed of its CUDA
// backend to M=1 specialised linears (a row-1 kernel and a split-K one) and
// switches to dense GEMMs for prefill.  On gfx950 the small-batch side is
// k_gemv: fp32 activations held in VGPRs, each weight row reduced by one
// 64-lane (or 32-lane) group with 16-byte non-temporal loads, no split-K
// partials (so no second pass), and an optional fused LayerNorm + token-shift
// prologue.  The MFMA GEMM for larger batches and prefill is in k_mm.hip.
#include "launch.h"

#include <stdio.h>
#include <type_traits>

// ============================================================== GEMV
// The fused LayerNorm prologue holds a lane's K slice of every row in VGPRs
// (B * NCH * 8 floats) and the mixed rows in LDS; it is instantiated only
// up to this many floats per lane.
constexpr int kFusedMaxFloats = 80;

// Epilogue family fixed at compile time (GV_MIXED reads it per segment);
// it also gives each projection class its own kernel symbol in traces.
// GV_PREV: the channel-mix key (EPI_PRE) followed by that workgroup's share
// of the sparse value projection: for each of its rows with h = relu(pre)^2
// > 0 in some batch row, h times the row's W_val row is added into a
// per-workgroup partial sum of the output, which k_cmix_fold adds up in a
// fixed order.  Only active value rows are read, and the value work no
// longer waits behind a separate compaction pass.
enum : int { GV_MIXED = 0, GV_PRE = 1, GV_RESID = 2, GV_NONE = 3, GV_PREV = 4 };

// Sum over each aligned group of LPR lanes (all lanes active): DPP moves for
// 16 and 64 lanes (an xor shuffle is an LDS permute), shuffles otherwise.
template <int LPR>
RW_DEV float group_sum(float v) {
  if constexpr (LPR == 64) {
    return wave_sum(v);
  } else if constexpr (LPR == 16) {
    return sum16(v);
  } else {
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
  }
}

// NWV waves per workgroup: 4, or 5 for launches with neither the fused
// LayerNorm prologue nor the value epilogue (both written for four waves).
// Q: the int8 route.  A weight byte u holds the code u - 128 of a symmetric
// per-row scale s, so a row's dot product is s (sum u x - 128 sum x): one
// unsigned-byte convert and one FMA per weight, as for fp16, at half the bytes.
template <int B, int LPR, int NCH, int RPW, int EPK, int NWV = 4, bool Q = false>
__global__ __launch_bounds__(64 * NWV) void k_gemv(ProjArgs a) {
  static_assert(NWV == 4 || EPK != GV_PREV, "the value epilogue assumes four waves");
  constexpr int GPW = 64 / LPR;
  constexpr int ROWS_WAVE = GPW * RPW;
  constexpr int ROWS_WG = NWV * ROWS_WAVE;
  constexpr int K = LPR * NCH * 8;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane / LPR;
  const int lig = lane % LPR;
  const int row_wg = blockIdx.x * ROWS_WG;
  const Seg sg = pick_seg(a, row_wg);
  const int row_base = row_wg + wave * ROWS_WAVE + grp * RPW;

  using WV = typename std::conditional<Q, u32x2, u32x4>::type;
  WV w[RPW][NCH];
  float wsc[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int row = row_base + i;
    if constexpr (Q) {
      const uint8_t* wp = a.Wq + (long)row * K + lig * 8;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (row < sg.row1)
          w[i][c] = ld8_nt(wp + c * LPR * 8);
        else
          w[i][c] = WV{0u, 0u};
      }
      wsc[i] = row < sg.row1 ? a.Wsc[row] : 0.0f;
    } else {
      const half_t* wp = a.W + (long)row * K + lig * 8;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (row < sg.row1)
          w[i][c] = ld16_nt(wp + c * LPR * 8);
        else
          w[i][c] = WV{0u, 0u, 0u, 0u};
      }
      wsc[i] = 1.0f;
    }
  }

  // Activations for this lane's K slice: k = (c * LPR + lig) * 8 + e.
  float xa[B][NCH][8];
  if (a.ln.mode == LNP_NONE) {
    const float* X = reinterpret_cast<const float*>(sg.act);
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const float* xp = X + (long)b * sg.ld_act + (c * LPR + lig) * 8;
        const floatx4 p0 = ldf4(xp), p1 = ldf4(xp + 4);
        xa[b][c][0] = p0.x; xa[b][c][1] = p0.y; xa[b][c][2] = p0.z; xa[b][c][3] = p0.w;
        xa[b][c][4] = p1.x; xa[b][c][5] = p1.y; xa[b][c][6] = p1.z; xa[b][c][7] = p1.w;
      }
  } else if constexpr (B * NCH <= kFusedMaxFloats / 8 && NWV == 4) {
    // Fused LayerNorm + token-shift mix, computed once per workgroup while
    // the weight loads above are in flight: wave w normalises the quarter
    // [w K/4, (w+1) K/4) of every row (coalesced, stride-64 lanes), row
    // statistics are combined through LDS, and the mixed row is shared
    // through LDS with every wave's K slice.
    constexpr int QK = K / 4;          // elements per wave
    constexpr int PER = QK / 64;       // per lane
    __shared__ __attribute__((aligned(16))) float s_xq[B][K];
    __shared__ float s_st[B][4][2];
    // every global load of the prologue is issued before the first barrier
    float xv[B][PER], gv[PER], bv[PER], mv[PER], pvv[B][PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int k = wave * QK + lane + 64 * j;
      gv[j] = a.ln.g[k];
      bv[j] = a.ln.b[k];
      mv[j] = a.ln.mode == LNP_MIX ? sg.mix[k] : 0.f;
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float* prev = nullptr;
      if (a.ln.mode == LNP_MIX) {
        const int slot = a.ln.slots[b];
        if (slot >= 0 && slot < a.ln.n_slots)
          prev = a.ln.pool + (long)slot * a.ln.slot_stride + a.ln.shift_off;
      }
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int k = wave * QK + lane + 64 * j;
        xv[b][j] = a.ln.x[(long)b * K + k];
        pvv[b][j] = prev ? prev[k] : 0.f;
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float sm = 0.f;
#pragma unroll
      for (int j = 0; j < PER; ++j) sm += xv[b][j];
      sm = wave_sum(sm);
      if (lane == 0) s_st[b][wave][0] = sm;
    }
    __syncthreads();
    float mean[B], rstd[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      mean[b] = (s_st[b][0][0] + s_st[b][1][0] + s_st[b][2][0] + s_st[b][3][0]) * (1.0f / K);
      float q = 0.f;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const float d = xv[b][j] - mean[b];
        q += d * d;
      }
      q = wave_sum(q);
      if (lane == 0) s_st[b][wave][1] = q;
    }
    __syncthreads();
    const bool writer = blockIdx.x == 0 && a.ln.u_out;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      rstd[b] = 1.0f / sqrtf((s_st[b][0][1] + s_st[b][1][1] + s_st[b][2][1] + s_st[b][3][1]) *
                                 (1.0f / K) + 1e-5f);
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int k = wave * QK + lane + 64 * j;
        const float u = (xv[b][j] - mean[b]) * rstd[b] * gv[j] + bv[j];
        if (writer) a.ln.u_out[(long)b * K + k] = u;
        s_xq[b][k] = a.ln.mode == LNP_MIX ? u + (pvv[b][j] - u) * mv[j] : u;
      }
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const float* xp = &s_xq[b][(c * LPR + lig) * 8];
        const floatx4 p0 = *reinterpret_cast<const floatx4*>(xp);
        const floatx4 p1 = *reinterpret_cast<const floatx4*>(xp + 4);
        xa[b][c][0] = p0.x; xa[b][c][1] = p0.y; xa[b][c][2] = p0.z; xa[b][c][3] = p0.w;
        xa[b][c][4] = p1.x; xa[b][c][5] = p1.y; xa[b][c][6] = p1.z; xa[b][c][7] = p1.w;
      }
  }

  float acc[RPW][B];
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[i][b] = 0.0f;

#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if constexpr (Q) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const unsigned word = e < 4 ? w[i][c].x : w[i][c].y;
          const float wf = (float)((word >> (8 * (e & 3))) & 0xFFu);
#pragma unroll
          for (int b = 0; b < B; ++b) acc[i][b] = fmaf(wf, xa[b][c][e], acc[i][b]);
        }
      } else {
        const half8 h = __builtin_bit_cast(half8, w[i][c]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float wf = (float)h[e];
#pragma unroll
          for (int b = 0; b < B; ++b) acc[i][b] = fmaf(wf, xa[b][c][e], acc[i][b]);
        }
      }
    }

#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[i][b] = group_sum<LPR>(acc[i][b]);

  if constexpr (Q) {
    // remove the byte bias with the group's activation sums, then scale the row
    float sx[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float t = 0.0f;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) t += xa[b][c][e];
      sx[b] = group_sum<LPR>(t);
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int b = 0; b < B; ++b) acc[i][b] = wsc[i] * fmaf(-128.0f, sx[b], acc[i][b]);
  }

  __shared__ float s_h[EPK == GV_PREV ? B : 1][EPK == GV_PREV ? ROWS_WG : 1];
  if constexpr (EPK == GV_PREV) {
    // rows past the end stay inactive
    if (threadIdx.x < B * ROWS_WG) s_h[threadIdx.x / ROWS_WG][threadIdx.x % ROWS_WG] = 0.0f;
    __syncthreads();
  }
  if (lig == 0) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int row = row_base + i;
      if (row < sg.row1) {
        const int n = row - sg.row0;
        const int epi = (EPK == GV_PRE || EPK == GV_PREV) ? EPI_PRE : EPK == GV_RESID ? EPI_RESID
                        : EPK == GV_NONE ? EPI_NONE : sg.epi;
        if (epi == EPI_PRE) {
          bool any = false;
#pragma unroll
          for (int b = 0; b < B; ++b) {
            const float pre = acc[i][b] + sg.aux[n];
            ((float*)sg.out)[(long)b * sg.ld_out + n] = pre;
            any |= pre > 0.0f;
            if constexpr (EPK == GV_PREV) s_h[b][row - row_wg] = pre > 0.0f ? pre * pre : 0.0f;
          }
          if (sg.mask) sg.mask[n] = any ? 1 : 0;
        } else {
#pragma unroll
          for (int b = 0; b < B; ++b) {
            float* o = (float*)sg.out + (long)b * sg.ld_out + n;
            if (epi == EPI_RESID)
              *o += acc[i][b];
            else if (epi == EPI_NONE)
              *o = acc[i][b];
            else
              epi_store(sg, n, b, acc[i][b]);
          }
        }
      }
    }
  }

  if constexpr (EPK == GV_PREV) {
    __syncthreads();
    // rows of this workgroup with any active batch row, as a bit set
    unsigned act = 0;
#pragma unroll
    for (int i = 0; i < ROWS_WG; ++i) {
      bool any = false;
#pragma unroll
      for (int b = 0; b < B; ++b) any |= s_h[b][i] > 0.0f;
      act |= any ? (1u << i) : 0u;
    }
    // thread t owns 8-column chunks t and t + 256 of the output row
    const int nchunk = a.vC / 8;
    const int c0 = threadIdx.x, c1 = threadIdx.x + 256;
    float pacc[B][2][8];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int e = 0; e < 8; ++e) { pacc[b][0][e] = 0.f; pacc[b][1][e] = 0.f; }
    float corr[B];   // int8 route: sum of h * s over the rows taken, times the bias 128
#pragma unroll
    for (int b = 0; b < B; ++b) corr[b] = 0.f;
    // up to VP active rows per pass, their loads issued together (only for
    // the pass's rows: the condition is the same in every thread; columns
    // past the row end re-read the last chunk and are not stored), so a
    // workgroup with up to VP active rows of its 20 (about 3 on average at
    // 85 % sparsity) makes one dependent round trip
    constexpr int VP = 12;
    const int c0l = c0 < nchunk ? c0 : nchunk - 1;
    const int c1l = c1 < nchunk ? c1 : nchunk - 1;
    while (act) {
      int rr[VP];
      int nr = 0;
#pragma unroll
      for (int u = 0; u < VP; ++u) {
        rr[u] = act ? __builtin_ctz(act) : 0;
        nr += act ? 1 : 0;
        act &= act - 1;
      }
#pragma unroll
      for (int u = 1; u < VP; ++u) rr[u] = u < nr ? rr[u] : rr[0];
      if constexpr (Q) {
        u32x2 q0[VP], q1[VP];
        float vs[VP];
#pragma unroll
        for (int u = 0; u < VP; ++u) {
          const uint8_t* wr = a.vWq + (long)(row_wg + rr[u]) * a.vC;
          q0[u] = u < nr ? ld8(wr + c0l * 8) : u32x2{0u, 0u};
          q1[u] = u < nr ? ld8(wr + c1l * 8) : u32x2{0u, 0u};
          vs[u] = u < nr ? a.vSc[row_wg + rr[u]] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < VP; ++u) {
          if (u < nr) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
              const float hs = s_h[b][rr[u]] * vs[u];
              corr[b] += hs;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const unsigned w0e = e < 4 ? q0[u].x : q0[u].y;
                const unsigned w1e = e < 4 ? q1[u].x : q1[u].y;
                pacc[b][0][e] = fmaf(hs, (float)((w0e >> (8 * (e & 3))) & 0xFFu), pacc[b][0][e]);
                pacc[b][1][e] = fmaf(hs, (float)((w1e >> (8 * (e & 3))) & 0xFFu), pacc[b][1][e]);
              }
            }
          }
        }
        continue;
      }
      u32x4 w0[VP], w1[VP];
#pragma unroll
      for (int u = 0; u < VP; ++u) {
        const half_t* wr = a.vW + (long)(row_wg + rr[u]) * a.vC;
        w0[u] = u < nr ? ld16(wr + c0l * 8) : u32x4{0u, 0u, 0u, 0u};
        w1[u] = u < nr ? ld16(wr + c1l * 8) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < VP; ++u) {
        if (u < nr) {
          const half8 h0 = __builtin_bit_cast(half8, w0[u]);
          const half8 h1 = __builtin_bit_cast(half8, w1[u]);
#pragma unroll
          for (int b = 0; b < B; ++b) {
            const float hb = s_h[b][rr[u]];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              pacc[b][0][e] = fmaf(hb, (float)h0[e], pacc[b][0][e]);
              pacc[b][1][e] = fmaf(hb, (float)h1[e], pacc[b][1][e]);
            }
          }
        }
      }
    }
    if constexpr (Q) {
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pacc[b][0][e] = fmaf(-128.0f, corr[b], pacc[b][0][e]);
          pacc[b][1][e] = fmaf(-128.0f, corr[b], pacc[b][1][e]);
        }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float* dst = a.vpart + ((long)blockIdx.x * B + b) * a.vC;
      if (c0 < nchunk) {
        stf4(dst + c0 * 8, floatx4{pacc[b][0][0], pacc[b][0][1], pacc[b][0][2], pacc[b][0][3]});
        stf4(dst + c0 * 8 + 4, floatx4{pacc[b][0][4], pacc[b][0][5], pacc[b][0][6], pacc[b][0][7]});
      }
      if (c1 < nchunk) {
        stf4(dst + c1 * 8, floatx4{pacc[b][1][0], pacc[b][1][1], pacc[b][1][2], pacc[b][1][3]});
        stf4(dst + c1 * 8 + 4, floatx4{pacc[b][1][4], pacc[b][1][5], pacc[b][1][6], pacc[b][1][7]});
      }
    }
  }
}

static constexpr int gemv_rpw(int B) { return B <= 2 ? 4 : 2; }

int gemv_rows_per_wg(int B, int K) {
  const int lpr = (K == 256) ? 32 : 64;
  return 4 * (64 / lpr) * gemv_rpw(B);
}

// Rows per workgroup of a launch.  Workgroups spread evenly over the 256 CUs,
// so the CU holding the most rows sets the time: a one-segment launch at B = 1
// takes 20-row workgroups (four waves of 5 rows) or, unless it needs four
// waves (fused prologue or value epilogue), 10-row ones (five waves of 2
// rows) when that lowers it (2.9B:
// the channel-mix key's 640 workgroups of 16 rows leave half the CUs three,
// 512 of 20 give every CU two; W_o's 160 workgroups leave 96 CUs idle, 256 of
// 10 fill them).  K = 2560 and 4096 only.
int gemv_launch_rows(int B, int K, int rows, int nseg, bool four_waves) {
  const int base = gemv_rows_per_wg(B, K);
  if (B != 1 || nseg != 1 || (K != 2560 && K != 4096)) return base;
  auto per_cu = [&](int r) { return rows % r ? 1 << 30 : (rows / r + 255) / 256 * r; };
  int best = base;
  if (per_cu(20) < per_cu(best)) best = 20;
  if (!four_waves && per_cu(10) < per_cu(best)) best = 10;
  return best;
}

bool gemv_supported(int B, int K) {
  if (B < 1 || B > 4) return false;
  if (K == 256) return true;
  return K % 512 == 0 && K / 512 >= 1 && K / 512 <= 8;
}

// The fused LayerNorm prologue keeps a lane's whole K slice of every row in
// VGPRs; bound that to 80 floats.
bool gemv_fused_ok(int B, int K) {
  if (!gemv_supported(B, K)) return false;
  const int nch = K == 256 ? 1 : K / 512;
  return B * nch <= kFusedMaxFloats / 8;
}

static int gemv_epk(const ProjArgs& a) {
  if (a.vW) return GV_PREV;
  int e = a.seg[0].epi;
  for (int i = 1; i < a.nseg; ++i)
    if (a.seg[i].epi != e) return GV_MIXED;
  return e == EPI_PRE ? GV_PRE : e == EPI_RESID ? GV_RESID : e == EPI_NONE ? GV_NONE : GV_MIXED;
}

template <int B, int LPR, int NCH, int RPW, int NWV = 4, bool Q = false>
static void gemv_launch_epk(int epk, dim3 grid, hipStream_t st, const ProjArgs& a) {
  const dim3 blk(64 * NWV);
  switch (epk) {
    case GV_PRE: hipLaunchKernelGGL((k_gemv<B, LPR, NCH, RPW, GV_PRE, NWV, Q>), grid, blk, 0, st, a); break;
    case GV_RESID: hipLaunchKernelGGL((k_gemv<B, LPR, NCH, RPW, GV_RESID, NWV, Q>), grid, blk, 0, st, a); break;
    case GV_NONE: hipLaunchKernelGGL((k_gemv<B, LPR, NCH, RPW, GV_NONE, NWV, Q>), grid, blk, 0, st, a); break;
    case GV_PREV:
      if constexpr (NWV == 4)
        hipLaunchKernelGGL((k_gemv<B, LPR, NCH, RPW, GV_PREV, NWV, Q>), grid, blk, 0, st, a);
      break;
    default: hipLaunchKernelGGL((k_gemv<B, LPR, NCH, RPW, GV_MIXED, NWV, Q>), grid, blk, 0, st, a); break;
  }
}

template <int B, bool Q = false>
static hipError_t gemv_dispatch_b(const ProjArgs& a, int total_rows, hipStream_t st) {
  constexpr int RPW = gemv_rpw(B);
  const int K = a.K;
  const int rows_wg = gemv_launch_rows(B, K, total_rows, a.nseg, a.ln.mode != LNP_NONE || a.vW != nullptr);
  const dim3 grid((total_rows + rows_wg - 1) / rows_wg);
  const int epk = gemv_epk(a);
  if constexpr (B == 1) {
    if (rows_wg == 20) {
      if (K == 2560) gemv_launch_epk<1, 64, 5, 5, 4, Q>(epk, grid, st, a);
      else gemv_launch_epk<1, 64, 8, 5, 4, Q>(epk, grid, st, a);
      return hipGetLastError();
    }
    if (rows_wg == 10) {   // five waves: no prologue, no value epilogue
      if (K == 2560) gemv_launch_epk<1, 64, 5, 2, 5, Q>(epk, grid, st, a);
      else gemv_launch_epk<1, 64, 8, 2, 5, Q>(epk, grid, st, a);
      return hipGetLastError();
    }
  }
  if (K == 256) {
    gemv_launch_epk<B, 32, 1, RPW, 4, Q>(epk, grid, st, a);
    return hipGetLastError();
  }
  switch (K / 512) {
#define CASE(n) case n: gemv_launch_epk<B, 64, n, RPW, 4, Q>(epk, grid, st, a); break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
#undef CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemv(const ProjArgs& a, int total_rows, hipStream_t st) {
  if (a.Wq) {
    if (a.vW && !a.vWq) return hipErrorInvalidValue;
    switch (a.M) {
      case 1: return gemv_dispatch_b<1, true>(a, total_rows, st);
      case 2: return gemv_dispatch_b<2, true>(a, total_rows, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.M) {
    case 1: return gemv_dispatch_b<1>(a, total_rows, st);
    case 2: return gemv_dispatch_b<2>(a, total_rows, st);
    case 3: return gemv_dispatch_b<3>(a, total_rows, st);
    case 4: return gemv_dispatch_b<4>(a, total_rows, st);
    default: return hipErrorInvalidValue;
  }
}

// Template arguments as a trace prints them, e.g. "k_gemv<1, 64, 5, 4, 1, 4, false>", for
// a launch of `rows` output rows in `nseg` segments (four_waves: it has the
// fused prologue or the value epilogue; q8: the int8 route).
const char* gemv_kernel_name(int B, int K, int epi, int rows, int nseg, bool four_waves, bool q8) {
  static char names[2][5][9][5][3][48];
  if (!gemv_supported(B, K)) return "k_gemv";
  const int lpr = K == 256 ? 32 : 64;
  const int nch = K == 256 ? 1 : K / 512;
  const int epk = epi == -2 ? GV_PREV : epi == EPI_PRE ? GV_PRE : epi == EPI_RESID ? GV_RESID
                  : epi == EPI_NONE ? GV_NONE : GV_MIXED;
  const int rw = gemv_launch_rows(B, K, rows, nseg, four_waves);
  char* s = names[q8 ? 1 : 0][B][nch][epk][rw == 20 ? 1 : rw == 10 ? 2 : 0];
  if (!s[0])
    snprintf(s, sizeof(names[0][0][0][0][0]), "k_gemv<%d, %d, %d, %d, %d, %d, %s>", B, lpr, nch,
             rw == 10 ? 2 : rw == 20 ? 5 : gemv_rpw(B), epk, rw == 10 ? 5 : 4, q8 ? "true" : "false");
  return s;
}
